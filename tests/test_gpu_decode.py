"""GPU parity of the decode path against the oracle, through the C ABI.

Sizes are small enough for the oracle to finish in seconds but span several
scoring chunks (1,024 keys), several selection slices (4,096 keys), ragged
tails and the degenerate cases (empty pool, budget covering the pool, a
single key, exact ties).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (assert_outputs_close, assert_scores_close,
                         assert_selection_near_ties)
from workloads import WORKLOADS, make_decode_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _buffers(hs2, inp, w, **kw):
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers

    args = dict(n_heads=w.n_heads, k_top=w.k_top, window=w.window, sm_scale=w.sm_scale,
                dtype=w.dtype)
    args.update(kw)
    return make_buffers(inp, **args)


def _oracle_scores(inp, w):
    return oracle.full_attn_scores(inp["q"], inp["k"], inp["ctx_len"], tile_q=1,
                                   sm_scale=w.sm_scale)


CASES = [
    ("f32_4k", "decode_f32_4k", dict(), [4096]),
    ("f32_ragged", "decode_f32_4k", dict(batch=3, n_heads=5), [3000, 1153, 77]),
    ("bf16_ragged", "decode_bf16_64k_b16", dict(batch=3), [9000, 4097, 1152]),
    ("bf16_h7", "decode_bf16_64k_b16", dict(batch=2, n_heads=7), [5000, 130]),
    ("bf16_h1", "decode_bf16_64k_b16", dict(batch=2, n_heads=1), [2049, 1]),
    ("bf16_clusters", "decode_bf16_256k_b4", dict(batch=2), [20000, 16384]),
]


@pytest.mark.parametrize("name,wname,over,ctx", CASES, ids=[c[0] for c in CASES])
def test_scores_match_oracle(hs2, name, wname, over, ctx):
    from kv_cache_reuse_hs2_amd.torch_api import run_scores

    w = WORKLOADS[wname].replace(**over)
    inp = make_decode_inputs(w, ctx_lens=ctx, capacity=max(ctx))
    buf = _buffers(hs2, inp, w)
    _say(f"scores {name} ctx={ctx} H={w.n_heads} dtype={w.dtype}")
    run_scores(buf)
    torch.cuda.synchronize()
    ref, _, lse = _oracle_scores(inp, w)
    assert_scores_close(buf.scores.cpu().numpy(), ref, inp["ctx_len"])
    np.testing.assert_allclose(buf.lse_full.cpu().numpy(), lse, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("name,wname,over,ctx", CASES, ids=[c[0] for c in CASES])
def test_select_bit_exact_on_oracle_scores(hs2, name, wname, over, ctx):
    from kv_cache_reuse_hs2_amd.torch_api import run_select, to_device

    w = WORKLOADS[wname].replace(**over)
    inp = make_decode_inputs(w, ctx_lens=ctx, capacity=max(ctx))
    ref, _, _ = _oracle_scores(inp, w)
    buf = _buffers(hs2, inp, w)
    _say(f"select {name} ctx={ctx}")
    run_select(buf, scores=to_device(ref))
    torch.cuda.synchronize()
    top, cnt = oracle.select_topk_window(ref, inp["ctx_len"], n_q=1, tile_q=1, k_top=w.k_top,
                                         window=w.window)
    np.testing.assert_array_equal(buf.top_cnt.cpu().numpy(), cnt)
    np.testing.assert_array_equal(buf.top_idx.cpu().numpy(), top)


def _select_on(hs2, scores, ctx, *, k_top=1024, window=128):
    """Run the GPU selector on a given fp32 score array; compare bit-exactly."""
    from kv_cache_reuse_hs2_amd import make_desc, hs2_select_topk_window, hs2_workspace_size
    from kv_cache_reuse_hs2_amd.torch_api import to_device

    bsz, _, cap = scores.shape
    d = make_desc(batch=bsz, n_heads=32, k_top=k_top, window=window)
    ws = torch.empty(hs2_workspace_size(d, cap), dtype=torch.uint8, device="cuda")
    ti = torch.empty((bsz, 1, max(k_top, 1)), dtype=torch.int32, device="cuda")
    tc = torch.empty((bsz, 1), dtype=torch.int32, device="cuda")
    ctx = np.asarray(ctx, dtype=np.int32)
    hs2_select_topk_window(d, to_device(scores), to_device(ctx), cap, ti, tc, ws)
    torch.cuda.synchronize()
    top, cnt = oracle.select_topk_window(scores, ctx, n_q=1, tile_q=1, k_top=k_top, window=window)
    np.testing.assert_array_equal(tc.cpu().numpy(), cnt)
    if k_top > 0:
        np.testing.assert_array_equal(ti.cpu().numpy(), top)
    return top, cnt


def test_select_edge_cases(hs2):
    rng = np.random.default_rng(21)
    cap = 9000
    # ctx 0, 1, window-sized, window+1, budget = pool, budget+1, ragged large
    ctx = [0, 1, 128, 129, 1152, 1153, 8999, 9000]
    s = rng.random((len(ctx), 1, cap), dtype=np.float32)
    _say("select edge ctx")
    _select_on(hs2, s, ctx)
    _say("select k_top=0 and window=0")
    _select_on(hs2, s, ctx, k_top=0)
    _select_on(hs2, s, ctx, window=0)
    _select_on(hs2, s, ctx, k_top=2048, window=2048)
    _select_on(hs2, s, ctx, k_top=1, window=1)


def test_select_ties(hs2):
    rng = np.random.default_rng(22)
    cap = 20000
    _say("select ties: all equal")
    eq = np.full((2, 1, cap), 0.125, dtype=np.float32)
    top, cnt = _select_on(hs2, eq, [cap, 7000])
    assert np.array_equal(top[0, 0], np.arange(1024))
    _say("select ties: few distinct values")
    few = rng.integers(0, 5, size=(3, 1, cap)).astype(np.float32) / 4
    _select_on(hs2, few, [cap, 15000, 3000])
    _say("select ties: zeros and one large value")
    z = np.zeros((1, 1, cap), dtype=np.float32)
    z[0, 0, 17] = 3.0
    _select_on(hs2, z, [cap])
    _say("select ties: values differing in the last bit")
    base = np.float32(0.001)
    near = (base.view(np.uint32) + rng.integers(0, 3, size=(2, 1, cap)).astype(np.uint32)).view(np.float32)
    _select_on(hs2, near, [cap, 12345])


@pytest.mark.parametrize("name,wname,over,ctx", CASES, ids=[c[0] for c in CASES])
def test_sparse_matches_oracle_on_oracle_selection(hs2, name, wname, over, ctx):
    from kv_cache_reuse_hs2_amd.torch_api import run_sparse, to_device

    w = WORKLOADS[wname].replace(**over)
    inp = make_decode_inputs(w, ctx_lens=ctx, capacity=max(ctx))
    ref, _, _ = _oracle_scores(inp, w)
    top, cnt = oracle.select_topk_window(ref, inp["ctx_len"], n_q=1, tile_q=1, k_top=w.k_top,
                                         window=w.window)
    buf = _buffers(hs2, inp, w)
    _say(f"sparse {name} ctx={ctx}")
    run_sparse(buf, top_idx=to_device(top), top_cnt=to_device(cnt))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["ctx_len"], top,
                                             cnt, tile_q=1, window=w.window, sm_scale=w.sm_scale)
    assert_outputs_close(buf.o.cpu().numpy(), o_ref, w.dtype)
    np.testing.assert_allclose(buf.lse.cpu().numpy(), lse_ref, rtol=1e-5, atol=1e-5)


def test_sparse_independent_query_and_small_budgets(hs2):
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_sparse, to_device

    w = WORKLOADS["decode_bf16_64k_b16"].replace(batch=2)
    inp = make_decode_inputs(w, ctx_lens=[3000, 40], capacity=3000)
    q2 = make_decode_inputs(w, seed=w.seed + 1, ctx_lens=[3000, 40], capacity=3000)
    for k_top, window in [(1024, 128), (7, 0), (0, 5), (1, 1), (2048, 2048)]:
        ref, _, _ = _oracle_scores(inp, w)
        top, cnt = oracle.select_topk_window(ref, inp["ctx_len"], n_q=1, tile_q=1, k_top=k_top,
                                             window=window)
        buf = make_buffers(inp, n_heads=32, k_top=k_top, window=window, sm_scale=w.sm_scale,
                           dtype="bf16")
        _say(f"sparse own query k_top={k_top} window={window}")
        run_sparse(buf, q=to_device(q2["q_raw"]), top_idx=to_device(top if k_top else
                                                                      np.zeros((2, 1, 1), np.int32)),
                   top_cnt=to_device(cnt))
        torch.cuda.synchronize()
        o_ref, _ = oracle.sparse_attention(q2["q"], inp["k"], inp["v"], inp["ctx_len"], top, cnt,
                                           tile_q=1, window=window, sm_scale=w.sm_scale)
        assert_outputs_close(buf.o.cpu().numpy(), o_ref, "bf16")


def test_sparse_f32_budgets(hs2):
    """fp32 sparse layer at the usual budget (36 segments of 32 keys, merged
    from registers) and at the largest (128 segments, merged in a loop)."""
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_sparse, to_device

    w = WORKLOADS["decode_f32_4k"].replace(batch=2)
    inp = make_decode_inputs(w, ctx_lens=[4096, 1000], capacity=4096)
    ref, _, _ = _oracle_scores(inp, w)
    for k_top, window in [(1024, 128), (2048, 2048), (2048, 100)]:
        top, cnt = oracle.select_topk_window(ref, inp["ctx_len"], n_q=1, tile_q=1, k_top=k_top,
                                             window=window)
        buf = make_buffers(inp, n_heads=w.n_heads, k_top=k_top, window=window,
                           sm_scale=w.sm_scale, dtype="f32")
        _say(f"fp32 sparse k_top={k_top} window={window}")
        run_sparse(buf, top_idx=to_device(top), top_cnt=to_device(cnt))
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["ctx_len"], top,
                                                 cnt, tile_q=1, window=window,
                                                 sm_scale=w.sm_scale)
        assert_outputs_close(buf.o.cpu().numpy(), o_ref, "f32")
        np.testing.assert_allclose(buf.lse.cpu().numpy(), lse_ref, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("name,wname,over,ctx", CASES, ids=[c[0] for c in CASES])
def test_decode_step_end_to_end(hs2, name, wname, over, ctx):
    from kv_cache_reuse_hs2_amd.torch_api import run_step

    w = WORKLOADS[wname].replace(**over)
    inp = make_decode_inputs(w, ctx_lens=ctx, capacity=max(ctx))
    buf = _buffers(hs2, inp, w)
    _say(f"step {name} ctx={ctx}")
    run_step(buf)
    torch.cuda.synchronize()
    ref, _, _ = _oracle_scores(inp, w)
    top, cnt = oracle.select_topk_window(ref, inp["ctx_len"], n_q=1, tile_q=1, k_top=w.k_top,
                                         window=w.window)
    tg, cg = buf.top_idx.cpu().numpy(), buf.top_cnt.cpu().numpy()
    assert_selection_near_ties(tg, cg, top, cnt, ref, inp["ctx_len"], n_q=1, tile_q=1,
                               window=w.window)
    for b, planted in enumerate(inp["planted"]):
        assert set(planted.tolist()) <= set(tg[b, 0, : cg[b, 0]].tolist())
    # The sparse output on the GPU's own selection.
    o_ref, _ = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["ctx_len"], tg, cg,
                                       tile_q=1, window=w.window, sm_scale=w.sm_scale)
    assert_outputs_close(buf.o.cpu().numpy(), o_ref, w.dtype)


def test_identical_keys_select_lowest_indices_end_to_end(hs2):
    # All scores are then bitwise equal on the GPU too, so the tie rule is
    # pinned end to end: T = [0, 1024).
    from kv_cache_reuse_hs2_amd.torch_api import run_step

    w = WORKLOADS["decode_bf16_64k_b16"].replace(batch=1, recipe="plain")
    inp = make_decode_inputs(w, ctx_lens=[6000], capacity=6000)
    inp["k_raw"][:] = inp["k_raw"][0, 0]
    inp["k"][:] = inp["k"][0, 0]
    buf = _buffers(hs2, inp, w)
    _say("identical keys step")
    run_step(buf)
    torch.cuda.synchronize()
    assert np.array_equal(buf.top_idx.cpu().numpy()[0, 0], np.arange(1024))
    s = buf.scores.cpu().numpy()[0, 0, :6000]
    assert np.all(s == s[0])


def test_step_is_deterministic(hs2):
    from kv_cache_reuse_hs2_amd.torch_api import run_step

    w = WORKLOADS["decode_bf16_256k_b4"].replace(batch=2)
    inp = make_decode_inputs(w, ctx_lens=[30000, 25000], capacity=30000)
    buf = _buffers(hs2, inp, w)
    _say("determinism x5")
    outs = []
    for _ in range(5):
        run_step(buf)
        torch.cuda.synchronize()
        outs.append((buf.scores.clone(), buf.top_idx.clone(), buf.o.clone()))
    for s, t, o in outs[1:]:
        assert torch.equal(s, outs[0][0]) and torch.equal(t, outs[0][1]) and torch.equal(o, outs[0][2])


@pytest.mark.parametrize("name,wname,over,ctx", CASES, ids=[c[0] for c in CASES])
def test_fused_step_equals_three_calls(hs2, name, wname, over, ctx):
    # hs2_decode_step must give bit-for-bit the outputs of the three calls.
    from kv_cache_reuse_hs2_amd.torch_api import run_fused_step, run_step

    w = WORKLOADS[wname].replace(**over)
    inp = make_decode_inputs(w, ctx_lens=ctx, capacity=max(ctx))
    buf = _buffers(hs2, inp, w)
    _say(f"fused vs three calls {name} ctx={ctx}")
    run_step(buf)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (buf.scores, buf.top_idx, buf.top_cnt, buf.o, buf.lse, buf.lse_full)]
    for t in (buf.scores, buf.top_idx, buf.top_cnt, buf.o, buf.lse, buf.lse_full):
        t.fill_(7)
    run_fused_step(buf)
    torch.cuda.synchronize()
    got = (buf.scores, buf.top_idx, buf.top_cnt, buf.o, buf.lse, buf.lse_full)
    for b, n in enumerate(ctx):  # scores beyond a sequence's context are not written
        assert torch.equal(ref[0][b, :, :n], got[0][b, :, :n])
    for a, b in zip(ref[1:], got[1:]):
        assert torch.equal(a, b)


def test_fused_step_with_own_sparse_query(hs2):
    from kv_cache_reuse_hs2_amd.torch_api import run_fused_step, to_device

    w = WORKLOADS["decode_bf16_256k_b4"].replace(batch=2)
    inp = make_decode_inputs(w, ctx_lens=[12000, 7000], capacity=12000)
    q2 = make_decode_inputs(w, seed=w.seed + 1, ctx_lens=[12000, 7000], capacity=12000)
    buf = _buffers(hs2, inp, w)
    _say("fused step with q_sparse")
    run_fused_step(buf, q_sparse=to_device(q2["q_raw"]))
    torch.cuda.synchronize()
    tg, cg = buf.top_idx.cpu().numpy(), buf.top_cnt.cpu().numpy()
    ref, _, _ = _oracle_scores(inp, w)
    top, cnt = oracle.select_topk_window(ref, inp["ctx_len"], n_q=1, tile_q=1, k_top=w.k_top,
                                         window=w.window)
    assert_selection_near_ties(tg, cg, top, cnt, ref, inp["ctx_len"], n_q=1, tile_q=1,
                               window=w.window)
    o_ref, _ = oracle.sparse_attention(q2["q"], inp["k"], inp["v"], inp["ctx_len"], tg, cg,
                                       tile_q=1, window=w.window, sm_scale=w.sm_scale)
    assert_outputs_close(buf.o.cpu().numpy(), o_ref, "bf16")
