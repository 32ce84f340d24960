"""The entry points replayed from HIP graphs give the eager results, bit for bit.

The benchmark times the decode step replayed from captured graphs, so every
replay must recompute everything: each test runs a call eagerly, clears the
outputs, captures the same call, and replays the graph three times with other
eager work and synchronisations in between, comparing every replay with the
eager result.  The kernels are deterministic (fixed reduction orders), and the
library clears its own workspace with kernels, not memsets.
"""

import sys

import pytest
import torch

from workloads import WORKLOADS, make_decode_inputs, make_prefill_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _snapshot(tensors):
    torch.cuda.synchronize()
    return [t.clone() for t in tensors]


def _fill(outputs):
    # A fixed non-NaN filler, so that entries a call leaves unwritten (scores
    # past a sequence's end) compare equal too.
    for t in outputs:
        t.fill_(-7)


def _check_replays(call, outputs, disturb, clear=_fill):
    """Eager reference, then three graph replays compared with it."""
    stream = torch.cuda.current_stream()
    clear(outputs)
    call()
    ref = _snapshot(outputs)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        call()  # warm-up on a side stream, as torch recommends before capture
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        clear(outputs)
        disturb()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outputs, ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager run"


def _decode_buffers(wname, over, ctx, **kw):
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers

    w = WORKLOADS[wname].replace(**over)
    inp = make_decode_inputs(w, ctx_lens=ctx, capacity=max(ctx))
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype, **kw)
    return w, inp, buf


@pytest.mark.parametrize("wname", ["decode_bf16_256k_b4", "decode_fp8_256k_b4"])
def test_decode_step_graph_replays(hs2, wname):
    from kv_cache_reuse_hs2_amd.torch_api import run_fused_step, run_scores

    _, _, buf = _decode_buffers(wname, dict(batch=3), [20000, 9000, 300])
    _, _, other = _decode_buffers(wname, dict(batch=2), [5000, 4097])
    _say(f"graph replays of the decode step ({wname})")
    outs = [buf.scores, buf.lse_full, buf.top_idx, buf.top_cnt, buf.o, buf.lse]
    _check_replays(lambda: run_fused_step(buf), outs, lambda: run_scores(other))


def test_three_calls_and_block_step_graph_replays(hs2):
    from kv_cache_reuse_hs2_amd.torch_api import run_fused_step_blocks, run_scores, run_step

    _, _, buf = _decode_buffers("decode_bf16_256k_b4", dict(batch=2), [12000, 7000])
    _, _, other = _decode_buffers("decode_bf16_256k_b4", dict(batch=2), [3000, 2000])
    _say("graph replays of the three-call step and the block-selection step")
    outs = [buf.scores, buf.lse_full, buf.top_idx, buf.top_cnt, buf.o, buf.lse]
    _check_replays(lambda: run_step(buf), outs, lambda: run_scores(other))
    _check_replays(lambda: run_fused_step_blocks(buf, 64), outs, lambda: run_scores(other))


def test_full_output_graph_replays(hs2):
    from kv_cache_reuse_hs2_amd.torch_api import run_scores, run_scores_full

    w, _, buf = _decode_buffers("decode_bf16_256k_b4", dict(batch=2), [15000, 4100])
    _, _, other = _decode_buffers("decode_bf16_256k_b4", dict(batch=1), [2500])
    o_full = torch.empty((w.batch, w.n_heads, 128), device="cuda")
    _say("graph replays of scoring with the full layer's output")
    _check_replays(lambda: run_scores_full(buf, o_full), [buf.scores, buf.lse_full, o_full],
                   lambda: run_scores(other))


def test_prefill_full_output_graph_replays(hs2):
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_scores, run_scores_full

    w = WORKLOADS["prefill_bf16_128k_8k"].replace(batch=2)
    inp = make_prefill_inputs(w, ctx_lens=[9000, 3000], n_q=128, capacity=9000)
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype="bf16", n_q=128, tile_q=64)
    _, _, other = _decode_buffers("decode_bf16_256k_b4", dict(batch=1), [3000])
    o_full = torch.empty((2, 128, w.n_heads, 128), device="cuda")
    _say("graph replays of prefill scoring with the full layer's output")
    _check_replays(lambda: run_scores_full(buf, o_full), [buf.scores, buf.lse_full, o_full],
                   lambda: run_scores(other))


def test_prefill_step_graph_replays(hs2):
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_fused_step, run_scores

    w = WORKLOADS["prefill_bf16_128k_8k"].replace(batch=1)
    inp = make_prefill_inputs(w, ctx_lens=[9000], n_q=128, capacity=9000)
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype="bf16", n_q=128, tile_q=64)
    _, _, other = _decode_buffers("decode_bf16_256k_b4", dict(batch=1), [3000])
    _say("graph replays of the prefill step")
    outs = [buf.scores, buf.lse_full, buf.top_idx, buf.top_cnt, buf.o, buf.lse]
    _check_replays(lambda: run_fused_step(buf), outs, lambda: run_scores(other))


def test_swa_and_bridge_decode_graph_replays(hs2):
    import kv_cache_reuse_hs2_amd as h
    from kv_cache_reuse_hs2_amd.torch_api import pack_bridge_weights

    g = torch.Generator(device="cuda").manual_seed(5)
    n_q, ctx, heads = 200, 1000, 32
    q = torch.randn((1, n_q, heads, 128), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((1, ctx, 128), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((1, ctx, 128), generator=g, device="cuda").to(torch.bfloat16)
    ctx_len = torch.tensor([ctx], dtype=torch.int32, device="cuda")
    o = torch.empty((1, n_q, heads, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, n_q, heads), device="cuda")
    desc = h.make_desc(batch=1, n_heads=heads, n_q=n_q, tile_q=1, k_top=0, window=128)
    junk = torch.empty(1 << 20, device="cuda")
    _say("graph replays of sliding-window attention")
    _check_replays(lambda: h.hs2_swa_attention(desc, q, k, v, ctx * 128, ctx_len, ctx, o,
                                               h.HS2_BF16, lse),
                   [o, lse], lambda: junk.normal_())
    dm, rows = 2048, 4
    hid = (torch.randn((rows, dm), generator=g, device="cuda") / dm ** 0.5).to(torch.bfloat16)
    wk = torch.randn((dm, 128), generator=g, device="cuda").to(torch.bfloat16)
    wv = torch.randn((dm, 128), generator=g, device="cuda").to(torch.bfloat16)
    wp = pack_bridge_weights(wk, wv, dm)
    kc = torch.zeros((rows, 64, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    pos = torch.tensor([0, 5, 63, 17], dtype=torch.int32, device="cuda")
    _say("graph replays of decode bridging")
    _check_replays(lambda: h.hs2_bridge_kv_decode(hid, dm, wp, rows, dm, pos, kc, vc, 64 * 128,
                                                  64),
                   [kc, vc], lambda: junk.normal_())
    assert int((kc != -7).sum()) == rows * 128  # exactly the four rows were written
