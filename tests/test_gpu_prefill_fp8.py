"""GPU parity of chunked prefill on an FP8 (E4M3) K/V cache against the oracle.

The pages quote prefill cost with an FP8 KV cache ("HySparse2: How Xiaomi
Split the Transformer to Fix Agent Prefill Costs", section "Results").  K and
V are E4M3 bytes with one fp32 scale per cache; the oracle decodes the same
bytes (``oracle.dequant_kv``) and runs the same definitions as for bf16, so
the bars are those of the bf16 prefill tests: scores element-wise 1e-4
relative, selection from GPU scores only at near-ties, sparse output max abs
2e-2 (relative L2 5e-3), log-sum-exp 1e-5, the full layer's own output
1e-4 of max|v| plus 2^-8 of sum_j p_j |v_j| (p enters P.V as bf16).  The shapes are the bf16 prefill test's seven (several key
splits and tiles, ragged batches, padded heads, tiles of 16/32/64, queries
before the cache start, a small pool) plus the 8,192-query prefill over a
131,072-token cache on a seeded sample of tiles.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (assert_outputs_close, assert_prefill_out_close, assert_scores_close,
                         assert_selection_near_ties)
from workloads import WORKLOADS, make_prefill_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _inputs(w, **kw):
    """Prefill inputs with E4M3 K/V; k and v are the oracle's decoding of the bytes."""
    inp = make_prefill_inputs(w, **kw)
    inp["k"] = oracle.dequant_kv(inp["k_raw"], inp["k_scale"])
    inp["v"] = oracle.dequant_kv(inp["v_raw"], inp["v_scale"])
    return inp


def _buffers(inp, w, n_q, tile_q):
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers

    return make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                        sm_scale=w.sm_scale, dtype="fp8", n_q=n_q, tile_q=tile_q)


CASES = [
    # name, batch, heads, ctx_lens, capacity, n_q, tile_q
    ("one_tile", 1, 32, [1200], 1200, 64, 64),
    ("two_tiles_splits", 1, 32, [20000], 20000, 128, 64),
    ("ragged_batch", 2, 32, [9000, 5000], 9008, 64, 64),
    ("heads7_tile16", 1, 7, [4000], 4000, 64, 16),
    ("tile32", 2, 32, [3100, 2600], 3104, 96, 32),
    ("before_cache_start", 1, 32, [40], 64, 64, 64),
    ("small_pool", 1, 32, [300], 304, 64, 64),
]


@pytest.mark.parametrize("name,bsz,heads,ctx,cap,n_q,tile_q", CASES, ids=[c[0] for c in CASES])
def test_fp8_prefill_matches_oracle(hs2, name, bsz, heads, ctx, cap, n_q, tile_q):
    from kv_cache_reuse_hs2_amd.torch_api import run_step

    w = WORKLOADS["prefill_fp8_128k_8k"].replace(batch=bsz, n_heads=heads)
    inp = _inputs(w, ctx_lens=ctx, n_q=n_q, capacity=cap)
    _say(f"fp8 prefill {name} ctx={ctx} n_q={n_q} tile={tile_q} H={heads}")
    buf = _buffers(inp, w, n_q, tile_q)
    run_step(buf)
    torch.cuda.synchronize()
    ref, _, lse = oracle.full_attn_scores(inp["q"], inp["k"], inp["ctx_len"], tile_q=tile_q,
                                          sm_scale=w.sm_scale)
    assert_scores_close(buf.scores.cpu().numpy(), ref, inp["ctx_len"])
    got_lse = buf.lse_full.cpu().numpy()
    fin = np.isfinite(lse)
    np.testing.assert_allclose(got_lse[fin], lse[fin], rtol=1e-5, atol=1e-5)
    assert np.all(np.isneginf(got_lse[~fin]))
    top, cnt = oracle.select_topk_window(ref, inp["ctx_len"], n_q=n_q, tile_q=tile_q,
                                         k_top=w.k_top, window=w.window)
    tg, cg = buf.top_idx.cpu().numpy(), buf.top_cnt.cpu().numpy()
    assert_selection_near_ties(tg, cg, top, cnt, ref, inp["ctx_len"], n_q=n_q, tile_q=tile_q,
                               window=w.window)
    o_ref, lse_ref = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["ctx_len"], tg, cg,
                                             tile_q=tile_q, window=w.window, sm_scale=w.sm_scale)
    assert_outputs_close(buf.o.cpu().numpy(), o_ref, "bf16")
    fin = np.isfinite(lse_ref)
    np.testing.assert_allclose(buf.lse.cpu().numpy()[fin], lse_ref[fin], rtol=1e-5, atol=1e-5)


def test_fp8_prefill_full_output(hs2):
    from kv_cache_reuse_hs2_amd.torch_api import run_scores, run_scores_full

    w = WORKLOADS["prefill_fp8_128k_8k"].replace(batch=2, n_heads=32)
    inp = _inputs(w, ctx_lens=[9000, 5000], n_q=64, capacity=9008)
    _say("fp8 prefill full output")
    buf = _buffers(inp, w, 64, 64)
    run_scores(buf)
    torch.cuda.synchronize()
    plain = buf.scores.clone()
    o_full = torch.full((2, 64, 32, 128), float("nan"), device="cuda")
    run_scores_full(buf, o_full)
    torch.cuda.synchronize()
    for b, n in enumerate(inp["ctx_len"]):
        assert torch.equal(buf.scores[b, :, :n], plain[b, :, :n])
    ref, o_ref, _ = oracle.full_attn_scores(inp["q"], inp["k"], inp["ctx_len"], tile_q=64,
                                            sm_scale=w.sm_scale, v=inp["v"])
    _, o_abs, _ = oracle.full_attn_scores(inp["q"], inp["k"], inp["ctx_len"], tile_q=64,
                                          sm_scale=w.sm_scale, v=np.abs(inp["v"]))
    assert_scores_close(buf.scores.cpu().numpy(), ref, inp["ctx_len"])
    assert_prefill_out_close(o_full.cpu().numpy().astype(np.float64), o_ref, o_abs,
                             np.abs(inp["v"]).max(), "fp8 prefill")


def test_fp8_prefill_fused_step_equals_three_calls(hs2):
    from kv_cache_reuse_hs2_amd.torch_api import run_fused_step, run_step

    w = WORKLOADS["prefill_fp8_128k_8k"].replace(batch=1)
    inp = _inputs(w, ctx_lens=[10000], n_q=128, capacity=10000)
    _say("fp8 prefill fused vs three calls")
    a = _buffers(inp, w, 128, 64)
    b = _buffers(inp, w, 128, 64)
    run_step(a)
    run_fused_step(b)
    torch.cuda.synchronize()
    assert torch.equal(a.scores[..., :10000], b.scores[..., :10000])
    for x, y in ((a.top_idx, b.top_idx), (a.top_cnt, b.top_cnt), (a.o, b.o), (a.lse, b.lse)):
        assert torch.equal(x, y)


def test_fp8_prefill_full_size_sampled_tiles(hs2):
    # 8,192 new queries appended to a 131,072-token E4M3 cache (139,264 keys),
    # 128 tiles of 64; the oracle checks a seeded sample of tiles, each with
    # the context that ends at its last query.
    from kv_cache_reuse_hs2_amd.torch_api import run_fused_step

    w = WORKLOADS["prefill_fp8_128k_8k"]
    inp = _inputs(w)
    n_q, tile_q, n = w.n_q, w.tile_q, w.ctx_len
    _say(f"fp8 prefill full size n_q={n_q} ctx={n}")
    buf = _buffers(inp, w, n_q, tile_q)
    run_fused_step(buf)
    torch.cuda.synchronize()
    scores = buf.scores.cpu().numpy()
    tg, cg, og = buf.top_idx.cpu().numpy(), buf.top_cnt.cpu().numpy(), buf.o.cpu().numpy()
    rng = np.random.default_rng(34)
    tiles = sorted(set([0, 127] + list(rng.integers(0, n_q // tile_q, 2))))
    for t in tiles:
        q0 = t * tile_q
        ctx_t = np.array([n - n_q + q0 + tile_q], dtype=np.int32)
        qs = inp["q"][:, q0:q0 + tile_q]
        ref, _, _ = oracle.full_attn_scores(qs, inp["k"][:, :ctx_t[0]], ctx_t, tile_q=tile_q,
                                            sm_scale=w.sm_scale)
        got = scores[:, t:t + 1, :]
        assert_scores_close(got, ref, ctx_t)
        top, cnt = oracle.select_topk_window(ref, ctx_t, n_q=tile_q, tile_q=tile_q,
                                             k_top=w.k_top, window=w.window)
        assert_selection_near_ties(tg[:, t:t + 1], cg[:, t:t + 1], top, cnt, ref, ctx_t,
                                   n_q=tile_q, tile_q=tile_q, window=w.window)
        o_ref, _ = oracle.sparse_attention(qs, inp["k"][:, :ctx_t[0]], inp["v"][:, :ctx_t[0]],
                                           ctx_t, tg[:, t:t + 1], cg[:, t:t + 1], tile_q=tile_q,
                                           window=w.window, sm_scale=w.sm_scale)
        assert_outputs_close(og[:, q0:q0 + tile_q], o_ref, "bf16")
        _say(f"tile {t} ok")
