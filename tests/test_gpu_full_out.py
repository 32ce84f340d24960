"""GPU parity of the full layer's own output (scoring with o_full).

The full-attention layer of a hybrid block produces its attention output
besides the selection ([Origins] "KV Reuse and Token-Level Sparse
Selection").  Decode: the second K pass also streams V and accumulates
sum_j p_hj v_j per 4,096-key chunk; the chunk partials are added in order.
Prefill: a third pass over K and V, exactly normalised with the first pass's
statistics, one workgroup per 8 queries over all their keys.

Bar: scores as without o_full (relative 1e-4).  Decode: o_full max
|gpu - oracle| <= 1e-4 * max|v|.  Both sides use the same stored bf16 (or
E4M3-widened) values; in decode p enters the MFMA as a bf16 high part plus a
bf16 low part (residual below 2^-17 relative), logits and sums are fp32, so
the error is some 1e-5 of the largest |v|, a tenth of the bar.  Prefill: the
output pass is bound by the matrix cores, and p enters its P.V MFMA rounded
once to bf16 (relative error at most 2^-8 per term), so each output may move
by 2^-8 * sum_j p_j |v_j| more; that sum is the oracle's output for |v|.  The
prefill outputs must also meet the bf16 path's bar: max abs error 2e-2 and
relative L2 error 5e-3.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_prefill_out_close, assert_scores_close
from workloads import WORKLOADS, make_decode_inputs, make_prefill_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _check(buf, o_full, inp, w):
    ref, o_ref, lse = oracle.full_attn_scores(inp["q"], inp["k"], inp["ctx_len"], tile_q=1,
                                              sm_scale=w.sm_scale, v=inp["v"])
    assert_scores_close(buf.scores.cpu().numpy(), ref, inp["ctx_len"])
    np.testing.assert_allclose(buf.lse_full.cpu().numpy(), lse, rtol=1e-5, atol=1e-5)
    got = o_full.cpu().numpy().astype(np.float64)
    want = o_ref[:, 0]
    vmax = max(np.abs(inp["v"]).max(), 1e-30)
    err = np.abs(got - want)
    assert err.max() <= 1e-4 * vmax, f"o_full max abs {err.max():.3e} (max|v| {vmax:.3e})"



CASES = [
    ("f32_4k", "decode_f32_4k", dict(), [4096]),
    ("f32_ragged_h5", "decode_f32_4k", dict(batch=3, n_heads=5), [3000, 1153, 77]),
    ("bf16_ragged", "decode_bf16_64k_b16", dict(batch=3), [9000, 4097, 1152]),
    ("bf16_h7", "decode_bf16_64k_b16", dict(batch=2, n_heads=7), [5000, 130]),
    ("bf16_h1_one_key", "decode_bf16_64k_b16", dict(batch=2, n_heads=1), [2049, 1]),
    ("bf16_clusters", "decode_bf16_256k_b4", dict(batch=2), [20000, 16384]),
    ("fp8_ragged", "decode_fp8_256k_b4", dict(batch=3), [9000, 4097, 1152]),
    ("fp8_h5", "decode_fp8_256k_b4", dict(batch=2, n_heads=5), [8193, 33]),
]


@pytest.mark.parametrize("name,wname,over,ctx", CASES, ids=[c[0] for c in CASES])
def test_full_output_matches_oracle(hs2, name, wname, over, ctx):
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_scores_full

    w = WORKLOADS[wname].replace(**over)
    inp = make_decode_inputs(w, ctx_lens=ctx, capacity=max(ctx))
    if w.dtype == "fp8":
        inp["k"] = oracle.dequant_kv(inp["k_raw"], inp["k_scale"])
        inp["v"] = oracle.dequant_kv(inp["v_raw"], inp["v_scale"])
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    o_full = torch.full((w.batch, w.n_heads, 128), float("nan"), device="cuda")
    _say(f"full output {name} ctx={ctx} H={w.n_heads} dtype={w.dtype}")
    run_scores_full(buf, o_full)
    torch.cuda.synchronize()
    _check(buf, o_full, inp, w)


def test_full_output_empty_sequence_is_zero(hs2):
    """A sequence with no keys has no attention mass: o_full 0, lse -inf."""
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_scores_full

    w = WORKLOADS["decode_bf16_64k_b16"].replace(batch=2)
    inp = make_decode_inputs(w, ctx_lens=[3000, 3000], capacity=3000)
    inp["ctx_len"] = np.array([3000, 0], dtype=np.int32)
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    o_full = torch.full((w.batch, w.n_heads, 128), float("nan"), device="cuda")
    _say("full output with an empty sequence")
    run_scores_full(buf, o_full)
    torch.cuda.synchronize()
    got = o_full.cpu().numpy()
    assert np.all(got[1] == 0.0)
    assert np.all(np.isneginf(buf.lse_full.cpu().numpy()[1]))
    _check(buf, o_full, inp, w)


def test_f32_scores_with_full_output_are_the_same_bits(hs2):
    """The fp32 path computes the importance with the same arithmetic either way."""
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_scores, run_scores_full

    w = WORKLOADS["decode_f32_4k"].replace(batch=2)
    inp = make_decode_inputs(w, ctx_lens=[4096, 2500], capacity=4096)
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    _say("fp32 scores with and without o_full")
    run_scores(buf)
    torch.cuda.synchronize()
    plain, lse = buf.scores.clone(), buf.lse_full.clone()
    o_full = torch.empty((w.batch, w.n_heads, 128), device="cuda")
    run_scores_full(buf, o_full)
    torch.cuda.synchronize()
    for b, n in enumerate(inp["ctx_len"]):
        assert torch.equal(buf.scores[b, :, :n], plain[b, :, :n])
    assert torch.equal(buf.lse_full, lse)


def test_scores_with_and_without_full_output_agree(hs2):
    """The o_full pass sums heads in another order: same scores to rounding."""
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_scores, run_scores_full

    w = WORKLOADS["decode_bf16_256k_b4"].replace(batch=2)
    inp = make_decode_inputs(w, ctx_lens=[12345, 8192], capacity=12345)
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    _say("scores with and without o_full")
    run_scores(buf)
    torch.cuda.synchronize()
    plain = buf.scores.clone()
    o_full = torch.empty((w.batch, w.n_heads, 128), device="cuda")
    run_scores_full(buf, o_full)
    torch.cuda.synchronize()
    a = plain.cpu().numpy()[:, :, :].astype(np.float64)
    bb = buf.scores.cpu().numpy().astype(np.float64)
    for b, n in enumerate(inp["ctx_len"]):
        np.testing.assert_allclose(bb[b, :, :n], a[b, :, :n], rtol=2e-6, atol=0)


PREFILL_CASES = [
    # name, batch, heads, ctx_lens, capacity, n_q, tile_q
    ("one_tile", 1, 32, [1200], 1200, 64, 64),
    ("two_tiles_splits", 1, 32, [20000], 20000, 128, 64),
    ("ragged_batch", 2, 32, [9000, 5000], 9000, 64, 64),
    ("heads7_tile16", 1, 7, [4000], 4000, 64, 16),
    ("heads1_tile32", 2, 1, [3100, 2600], 3100, 96, 32),
    ("before_cache_start", 1, 32, [40], 64, 64, 64),
    ("one_key", 1, 5, [1], 64, 16, 16),
]


def _prefill_buffers(name, bsz, heads, ctx, cap, n_q, tile_q):
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers

    w = WORKLOADS["prefill_bf16_128k_8k"].replace(batch=bsz, n_heads=heads)
    inp = make_prefill_inputs(w, ctx_lens=ctx, n_q=n_q, capacity=cap)
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype="bf16", n_q=n_q, tile_q=tile_q)
    return w, inp, buf


@pytest.mark.parametrize("name,bsz,heads,ctx,cap,n_q,tile_q", PREFILL_CASES,
                         ids=[c[0] for c in PREFILL_CASES])
def test_prefill_full_output_matches_oracle(hs2, name, bsz, heads, ctx, cap, n_q, tile_q):
    from kv_cache_reuse_hs2_amd.torch_api import run_scores, run_scores_full

    w, inp, buf = _prefill_buffers(name, bsz, heads, ctx, cap, n_q, tile_q)
    _say(f"prefill full output {name} ctx={ctx} n_q={n_q} tile={tile_q} H={heads}")
    run_scores(buf)
    torch.cuda.synchronize()
    plain, plain_lse = buf.scores.clone(), buf.lse_full.clone()
    o_full = torch.full((bsz, n_q, heads, 128), float("nan"), device="cuda")
    run_scores_full(buf, o_full)
    torch.cuda.synchronize()
    # the scores come from the same passes with or without o_full
    for b, n in enumerate(inp["ctx_len"]):
        assert torch.equal(buf.scores[b, :, :n], plain[b, :, :n])
    assert torch.equal(buf.lse_full, plain_lse)
    ref, o_ref, lse = oracle.full_attn_scores(inp["q"], inp["k"], inp["ctx_len"], tile_q=tile_q,
                                              sm_scale=w.sm_scale, v=inp["v"])
    _, o_abs, _ = oracle.full_attn_scores(inp["q"], inp["k"], inp["ctx_len"], tile_q=tile_q,
                                          sm_scale=w.sm_scale, v=np.abs(inp["v"]))
    assert_scores_close(buf.scores.cpu().numpy(), ref, inp["ctx_len"])
    got = o_full.cpu().numpy().astype(np.float64)
    vmax = max(np.abs(inp["v"]).max(), 1e-30)
    assert_prefill_out_close(got, o_ref, o_abs, vmax, name)
    # queries before the cache start see no key: output exactly 0
    dead = ~np.isfinite(lse)
    assert np.all(got[dead] == 0.0)


def test_prefill_full_output_full_size_sampled(hs2):
    """8,192 new queries on a 131,072-token cache (139,264 keys), the shape the
    benchmark times: a seeded sample of 16-query blocks is checked against the
    oracle, each with the context that ends at its last query (its queries see
    exactly those keys)."""
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_scores_full

    w = WORKLOADS["prefill_bf16_128k_8k"]
    inp = make_prefill_inputs(w)
    n_q, n = w.n_q, w.ctx_len
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype="bf16", n_q=n_q, tile_q=w.tile_q)
    o_full = torch.full((1, n_q, w.n_heads, 128), float("nan"), device="cuda")
    _say(f"prefill full output at full size n_q={n_q} ctx={n}")
    run_scores_full(buf, o_full)
    torch.cuda.synchronize()
    got_all = o_full.cpu().numpy()
    vmax = max(np.abs(inp["v"]).max(), 1e-30)
    rng = np.random.default_rng(41)
    blocks = sorted(set([0, 1, 255, 511] + list(rng.integers(0, n_q // 16, 2))))
    for blk in blocks:
        q0 = 16 * blk
        ctx_t = np.array([n - n_q + q0 + 16], dtype=np.int32)
        _, o_ref, _ = oracle.full_attn_scores(inp["q"][:, q0:q0 + 16], inp["k"][:, :ctx_t[0]],
                                              ctx_t, tile_q=16, sm_scale=w.sm_scale,
                                              v=inp["v"][:, :ctx_t[0]])
        _, o_abs, _ = oracle.full_attn_scores(inp["q"][:, q0:q0 + 16], inp["k"][:, :ctx_t[0]],
                                              ctx_t, tile_q=16, sm_scale=w.sm_scale,
                                              v=np.abs(inp["v"][:, :ctx_t[0]]))
        assert_prefill_out_close(got_all[:, q0:q0 + 16].astype(np.float64), o_ref, o_abs, vmax,
                           f"block {blk}")
