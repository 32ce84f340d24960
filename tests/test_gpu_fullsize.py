"""GPU parity at the measured decode shapes, in the launch configuration the
benchmark times (same entry points, same workspace, one stream).

The oracle computes every score, the selection and the sparse output of
these shapes in seconds, so the comparison is complete, not sampled.
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


def _run_full(name, **over):
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_select, run_step, to_device

    w = WORKLOADS[name].replace(**over)
    inp = make_decode_inputs(w)
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    print(f"[gpu] full-size step {name} B={w.batch} N={w.ctx_len}", flush=True)
    sys.stdout.flush()
    run_step(buf)
    torch.cuda.synchronize()
    scores = buf.scores.cpu().numpy()
    tg, cg, og = buf.top_idx.cpu().numpy(), buf.top_cnt.cpu().numpy(), buf.o.cpu().numpy()

    ref, _, _ = oracle.full_attn_scores(inp["q"], inp["k"], inp["ctx_len"], tile_q=1,
                                        sm_scale=w.sm_scale)
    assert_scores_close(scores, ref, inp["ctx_len"])
    top, cnt = oracle.select_topk_window(ref, inp["ctx_len"], n_q=1, tile_q=1, k_top=w.k_top,
                                         window=w.window)
    swaps = assert_selection_near_ties(tg, cg, top, cnt, ref, inp["ctx_len"], n_q=1, tile_q=1,
                                       window=w.window)
    print(f"[gpu] near-tie swaps: {swaps}", flush=True)
    for b, planted in enumerate(inp["planted"]):
        assert set(planted.tolist()) <= set(tg[b, 0, : cg[b, 0]].tolist())
    o_ref, _ = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["ctx_len"], tg, cg,
                                       tile_q=1, window=w.window, sm_scale=w.sm_scale)
    assert_outputs_close(og, o_ref, w.dtype)

    # The selector fed the oracle's own scores must agree bit for bit.
    print(f"[gpu] full-size select on oracle scores {name}", flush=True)
    run_select(buf, scores=to_device(ref))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(buf.top_cnt.cpu().numpy(), cnt)
    np.testing.assert_array_equal(buf.top_idx.cpu().numpy(), top)
    return w, inp, buf


def test_decode_256k_batch4_clusters(hs2):
    _run_full("decode_bf16_256k_b4")


def test_decode_64k_batch16_needles(hs2):
    _run_full("decode_bf16_64k_b16")


def test_decode_1m_context(hs2):
    # The decode half of the bridge workload: one sequence of 1,048,576 keys.
    _run_full("bridge_decode_bf16_1m", recipe="plain")


@pytest.mark.timeout(400)
def test_decode_max_capacity_4m(hs2):
    # The largest supported cache: one sequence of 4,194,304 keys (1 GiB of
    # bf16 K), through the three calls, and the full layer's own output.
    from kv_cache_reuse_hs2_amd.torch_api import run_scores_full

    w, inp, buf = _run_full("bridge_decode_bf16_1m", recipe="plain", ctx_len=4194304)
    o_full = torch.empty((1, w.n_heads, 128), device="cuda")
    print("[gpu] full output at 4,194,304 keys", flush=True)
    run_scores_full(buf, o_full)
    torch.cuda.synchronize()
    ref, o_ref, _ = oracle.full_attn_scores(inp["q"], inp["k"], inp["ctx_len"], tile_q=1,
                                            sm_scale=w.sm_scale, v=inp["v"])
    assert_scores_close(buf.scores.cpu().numpy(), ref, inp["ctx_len"])
    err = np.abs(o_full.cpu().numpy().astype(np.float64) - o_ref[:, 0]).max()
    assert err <= 1e-4 * np.abs(inp["v"]).max(), f"o_full max abs {err:.3e}"
