"""Seeded input generators (no method arithmetic; see the package docstring)."""

from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, storage type and generator recipe."""

    name: str
    kind: str            # "decode" | "prefill" | "bridge_decode"
    batch: int
    n_heads: int
    head_dim: int
    ctx_len: int         # keys in the cache, the new queries' own keys included
    n_q: int             # new queries per sequence (1 for decode)
    tile_q: int          # queries per selection group (1 for decode)
    k_top: int
    window: int
    dtype: str           # "f32" | "bf16" | "fp8": storage type of q, k, v (fp8: k, v
                         # in E4M3 with one scale per cache, q in bf16)
    seed: int
    recipe: str          # "needles" | "clusters" | "plain" | "bridge"
    n_needles: int = 0
    d_model: int = 0     # bridge only

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The measured shapes.  Sizes follow the contexts the pages use (32k
# pretraining, 256k post-training, 1M in the cost analysis) and the 1,024 +
# 128 selection budget.
WORKLOADS = {
    "decode_f32_4k": Workload(
        "decode_f32_4k", "decode", batch=1, n_heads=16, head_dim=128,
        ctx_len=4096, n_q=1, tile_q=1, k_top=1024, window=128, dtype="f32",
        seed=1001, recipe="needles", n_needles=8),
    "decode_bf16_64k_b16": Workload(
        "decode_bf16_64k_b16", "decode", batch=16, n_heads=32, head_dim=128,
        ctx_len=65536, n_q=1, tile_q=1, k_top=1024, window=128, dtype="bf16",
        seed=1002, recipe="needles", n_needles=32),
    "prefill_bf16_128k_8k": Workload(
        "prefill_bf16_128k_8k", "prefill", batch=1, n_heads=32, head_dim=128,
        ctx_len=131072 + 8192, n_q=8192, tile_q=64, k_top=1024, window=128,
        dtype="bf16", seed=1003, recipe="plain"),
    "decode_bf16_256k_b4": Workload(
        "decode_bf16_256k_b4", "decode", batch=4, n_heads=32, head_dim=128,
        ctx_len=262144, n_q=1, tile_q=1, k_top=1024, window=128, dtype="bf16",
        seed=1004, recipe="clusters"),
    "prefill_fp8_128k_8k": Workload(
        "prefill_fp8_128k_8k", "prefill", batch=1, n_heads=32, head_dim=128,
        ctx_len=131072 + 8192, n_q=8192, tile_q=64, k_top=1024, window=128,
        dtype="fp8", seed=1007, recipe="plain"),
    "decode_fp8_256k_b4": Workload(
        "decode_fp8_256k_b4", "decode", batch=4, n_heads=32, head_dim=128,
        ctx_len=262144, n_q=1, tile_q=1, k_top=1024, window=128, dtype="fp8",
        seed=1006, recipe="clusters"),
    "bridge_decode_bf16_1m": Workload(
        "bridge_decode_bf16_1m", "bridge_decode", batch=1, n_heads=32,
        head_dim=128, ctx_len=1048576, n_q=1, tile_q=1, k_top=1024, window=128,
        dtype="bf16", seed=1005, recipe="bridge", d_model=2048),
}

# Cluster sizes of the 256k workload: 262 keys (0.1% of 262,144) in 8 groups.
CLUSTER_SIZES = (33, 33, 33, 33, 33, 33, 32, 32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the exactly equal fp32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _store(x: np.ndarray, dtype: str):
    """Round an fp32 draw to the storage type: (values as fp32, raw array)."""
    if dtype == "f32":
        x = np.ascontiguousarray(x, dtype=np.float32)
        return x, x
    bits = bf16_bits(x)
    return bf16_bits_to_f32(bits), bits


def e4m3_codes(x: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """Quantise an fp32 array to FP8 E4M3 bytes with one scale: the scale maps
    the largest magnitude to 448 (the largest finite E4M3 value) and the
    scaled values are rounded to nearest, ties to even, by torch's float8
    conversion.  Returns (codes uint8, scale float32)."""
    import torch

    amax = float(np.max(np.abs(x)))
    scale = np.float32(amax / 448.0 if amax > 0 else 1.0)
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32) / scale)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy(), scale


def _unit(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def make_decode_inputs(w: Workload, *, seed: int | None = None,
                       ctx_lens=None, capacity: int | None = None) -> dict:
    """Decode inputs: q [B][1][H][D], k/v [B][cap][D], planted keys.

    ``ctx_lens`` (per sequence) and ``capacity`` may shrink or vary the
    sequences for parity tests; by default every sequence holds ``ctx_len``
    keys.  Returned dict: q, k, v (fp32 values equal to the stored ones),
    q_raw, k_raw, v_raw (fp32 arrays or bfloat16 bits), ctx_len int32 [B],
    planted (list of int64 position arrays per sequence).

    Recipes:
    * "needles": Q, K, V ~ N(0, s^2) with s = 1/sqrt(D) for fp32 storage and
      s = 1 for bfloat16; n_needles keys per sequence at distinct pool
      positions are set to 4 * rho * u_b, where u_b is the unit vector along
      the sum of the sequence's query heads and rho = s * sqrt(D) is the
      expected background key norm.
    * "clusters": Q, V ~ N(0, 1), K background ~ N(0, 1); 262 keys per
      sequence at distinct pool positions form 8 clusters: centre
      c_m = unit(u_b + g_m) with g_m ~ N(0, I/D), member
      sqrt(D) * unit(c_m + 0.05 e) with e ~ N(0, I/D).
    * "plain" / "bridge": Q, K, V ~ N(0, 1), nothing planted.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    bsz, n_heads, head_dim = w.batch, w.n_heads, w.head_dim
    cap = int(capacity if capacity is not None else w.ctx_len)
    if ctx_lens is None:
        ctx_lens = [min(w.ctx_len, cap)] * bsz
    ctx_len = np.asarray(ctx_lens, dtype=np.int32)
    assert ctx_len.shape == (bsz,) and np.all(ctx_len <= cap)
    scale = 1.0 / math.sqrt(head_dim) if w.dtype == "f32" and w.recipe == "needles" else 1.0

    q = rng.standard_normal((bsz, w.n_q, n_heads, head_dim), dtype=np.float32) * np.float32(scale)
    k = rng.standard_normal((bsz, cap, head_dim), dtype=np.float32) * np.float32(scale)
    v = rng.standard_normal((bsz, cap, head_dim), dtype=np.float32) * np.float32(scale)
    q_val, q_raw = _store(q, "bf16" if w.dtype == "fp8" else w.dtype)

    planted = []
    for b in range(bsz):
        pool = max(0, int(ctx_len[b]) - w.window)        # decode pool end
        u_b = _unit(q_val[b, 0].astype(np.float64).sum(axis=0))
        if w.recipe == "needles" and pool > 0:
            n = min(w.n_needles, pool)
            pos = np.sort(rng.choice(pool, size=n, replace=False))
            rho = scale * math.sqrt(head_dim)
            k[b, pos] = (4.0 * rho * u_b).astype(np.float32)
            planted.append(pos.astype(np.int64))
        elif w.recipe == "clusters" and pool > 0:
            n = min(sum(CLUSTER_SIZES), pool)
            pos = rng.choice(pool, size=n, replace=False)
            off = 0
            for size in CLUSTER_SIZES:
                members = pos[off:off + size]
                off += size
                g = rng.standard_normal(head_dim) / math.sqrt(head_dim)
                centre = _unit(u_b + g)
                e = rng.standard_normal((members.size, head_dim)) / math.sqrt(head_dim)
                k[b, members] = (math.sqrt(head_dim) * _unit(centre + 0.05 * e)).astype(np.float32)
                if off >= n:
                    break
            planted.append(np.sort(pos).astype(np.int64))
        else:
            planted.append(np.zeros(0, dtype=np.int64))

    if w.dtype == "fp8":
        # K and V as E4M3 bytes with one scale each; their values are left to
        # the consumer (the oracle decodes the bytes itself).
        k_raw, k_scale = e4m3_codes(k)
        v_raw, v_scale = e4m3_codes(v)
        return dict(q=q_val, k=None, v=None, q_raw=q_raw, k_raw=k_raw, v_raw=v_raw,
                    k_scale=k_scale, v_scale=v_scale, ctx_len=ctx_len, planted=planted,
                    capacity=cap)
    k_val, k_raw = _store(k, w.dtype)
    v_val, v_raw = _store(v, w.dtype)
    return dict(q=q_val, k=k_val, v=v_val, q_raw=q_raw, k_raw=k_raw,
                v_raw=v_raw, ctx_len=ctx_len, planted=planted, capacity=cap)


def make_prefill_inputs(w: Workload, *, seed: int | None = None,
                        ctx_lens=None, n_q: int | None = None,
                        capacity: int | None = None) -> dict:
    """Chunked-prefill inputs: q [B][n_q][H][D], k/v [B][cap][D], all N(0, 1).

    The n_q new queries are the last n_q positions of each sequence; their
    own keys are already in the cache.
    """
    n_q = int(n_q if n_q is not None else w.n_q)
    w = w.replace(n_q=n_q, recipe="plain")
    return make_decode_inputs(w, seed=seed, ctx_lens=ctx_lens, capacity=capacity)


def make_bridge_inputs(w: Workload, *, seed: int | None = None,
                       rows: int | None = None, row_chunk: int = 65536) -> dict:
    """KV Bridging inputs: hidden states H [M][d_model] ~ N(0, 1/d_model) and
    projection weights W_K, W_V [d_model][D] ~ N(0, 1), all stored in
    bfloat16, plus the decode query q [1][1][H][D] ~ N(0, 1).

    Draw order: q, W_K, W_V, then H in row chunks (so a 1M-row H never needs
    an fp32 copy in memory).  Returns bits (uint16) for h, w_k, w_v, q and the
    fp32 values of w_k, w_v, q; H's fp32 values are produced on demand with
    ``bf16_bits_to_f32``.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    m_rows = int(rows if rows is not None else w.ctx_len)
    d_model, head_dim = w.d_model, w.head_dim
    q = rng.standard_normal((1, 1, w.n_heads, head_dim), dtype=np.float32)
    wk = rng.standard_normal((d_model, head_dim), dtype=np.float32)
    wv = rng.standard_normal((d_model, head_dim), dtype=np.float32)
    h_bits = np.empty((m_rows, d_model), dtype=np.uint16)
    hs = np.float32(1.0 / math.sqrt(d_model))
    for r0 in range(0, m_rows, row_chunk):
        r1 = min(m_rows, r0 + row_chunk)
        h_bits[r0:r1] = bf16_bits(rng.standard_normal((r1 - r0, d_model), dtype=np.float32) * hs)
    q_val, q_bits = _store(q, "bf16")
    wk_val, wk_bits = _store(wk, "bf16")
    wv_val, wv_bits = _store(wv, "bf16")
    return dict(q=q_val, q_raw=q_bits, w_k=wk_val, w_k_raw=wk_bits, w_v=wv_val,
                w_v_raw=wv_bits, h_raw=h_bits, rows=m_rows)
