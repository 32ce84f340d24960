"""Padded caches: a per-sequence stride beyond the capacity, and NaN in every
cache row a call must not read (rows at or past a sequence's ctx_len, and the
padding), give results bit-identical to the same call on a dense cache.

This checks that every kernel addresses sequence b at b * kv_stride and keeps
its reads (clamped loads, staged bands, gathers, rings) inside [0, ctx_len[b]):
a single NaN read would reach the outputs through a dot product or a max.
"""

import sys

import numpy as np
import pytest
import torch

from workloads import WORKLOADS, make_decode_inputs, make_prefill_inputs

pytestmark = pytest.mark.gpu

PAD_ROWS = 72


def _say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _padded(t: torch.Tensor, ctx, nan_code: int) -> torch.Tensor:
    """[B][cap][D] cache -> [B][cap + PAD_ROWS][D] with the rows at or past each
    sequence's ctx_len (and the padding) set to a NaN code."""
    bsz, cap, d = t.shape
    out = torch.full((bsz, cap + PAD_ROWS, d), nan_code, dtype=t.dtype, device=t.device)
    for b, n in enumerate(ctx):
        out[b, :n] = t[b, :n]
    return out


def _nan_code(t: torch.Tensor) -> int:
    # bf16 bits 0x7FC0 (quiet NaN); E4M3 byte 0x7F (S.1111.111)
    return 0x7F if t.element_size() == 1 else 0x7FC0


def _pad_buffers(buf, ctx):
    code = _nan_code(buf.k)
    buf.k = _padded(buf.k, ctx, code)
    buf.v = _padded(buf.v, ctx, code)
    return buf


def _outs(buf):
    return [buf.scores, buf.lse_full, buf.top_idx, buf.top_cnt, buf.o, buf.lse]


def _same(a_list, b_list, ctx_of_scores=None):
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(a_list, b_list)):
        if i == 0 and ctx_of_scores is not None:  # scores: rows past ctx are not written
            for bb, n in enumerate(ctx_of_scores):
                assert torch.equal(a[bb, :, :n], b[bb, :, :n]), f"scores of sequence {bb} differ"
        else:
            assert torch.equal(a, b), f"output {i} differs"


@pytest.mark.parametrize("wname", ["decode_bf16_256k_b4", "decode_fp8_256k_b4"])
def test_decode_step_padded_cache(hs2, wname):
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_fused_step, run_fused_step_blocks

    ctx = [9000, 4097, 300]
    w = WORKLOADS[wname].replace(batch=3)
    inp = make_decode_inputs(w, ctx_lens=ctx, capacity=max(ctx))
    mk = lambda: make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,  # noqa: E731
                              sm_scale=w.sm_scale, dtype=w.dtype)
    dense, padded = mk(), _pad_buffers(mk(), ctx)
    assert padded.kv_stride == (max(ctx) + PAD_ROWS) * 128
    _say(f"decode step on a padded cache ({wname})")
    run_fused_step(dense)
    run_fused_step(padded)
    _same(_outs(padded), _outs(dense), ctx)
    _say(f"block-selection step on a padded cache ({wname})")
    run_fused_step_blocks(dense, 64)
    run_fused_step_blocks(padded, 64)
    _same(_outs(padded), _outs(dense), ctx)


def test_full_output_padded_cache(hs2):
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_scores_full

    ctx = [12000, 5000]
    w = WORKLOADS["decode_bf16_256k_b4"].replace(batch=2)
    inp = make_decode_inputs(w, ctx_lens=ctx, capacity=max(ctx))
    mk = lambda: make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,  # noqa: E731
                              sm_scale=w.sm_scale, dtype=w.dtype)
    dense, padded = mk(), _pad_buffers(mk(), ctx)
    o_d = torch.empty((2, w.n_heads, 128), device="cuda")
    o_p = torch.empty_like(o_d)
    _say("scoring with the full layer's output on a padded cache")
    run_scores_full(dense, o_d)
    run_scores_full(padded, o_p)
    _same([padded.scores, padded.lse_full, o_p], [dense.scores, dense.lse_full, o_d], ctx)


def test_prefill_step_padded_cache(hs2):
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_fused_step

    ctx = [7000, 2600]
    w = WORKLOADS["prefill_bf16_128k_8k"].replace(batch=2)
    inp = make_prefill_inputs(w, ctx_lens=ctx, n_q=128, capacity=max(ctx))
    mk = lambda: make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,  # noqa: E731
                              sm_scale=w.sm_scale, dtype="bf16", n_q=128, tile_q=64)
    dense, padded = mk(), _pad_buffers(mk(), ctx)
    _say("prefill step on a padded cache")
    run_fused_step(dense)
    run_fused_step(padded)
    _same(_outs(padded), _outs(dense), ctx)


def test_prefill_full_output_padded_cache(hs2):
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_scores_full

    ctx = [7000, 2600]
    w = WORKLOADS["prefill_bf16_128k_8k"].replace(batch=2)
    inp = make_prefill_inputs(w, ctx_lens=ctx, n_q=128, capacity=max(ctx))
    mk = lambda: make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,  # noqa: E731
                              sm_scale=w.sm_scale, dtype="bf16", n_q=128, tile_q=64)
    dense, padded = mk(), _pad_buffers(mk(), ctx)
    o_d = torch.empty((2, 128, w.n_heads, 128), device="cuda")
    o_p = torch.empty_like(o_d)
    _say("prefill scoring with the full layer's output on a padded cache")
    run_scores_full(dense, o_d)
    run_scores_full(padded, o_p)
    _same([padded.scores, padded.lse_full, o_p], [dense.scores, dense.lse_full, o_d], ctx)


@pytest.mark.parametrize("window", [128, 300])
def test_swa_padded_cache(hs2, window):
    import kv_cache_reuse_hs2_amd as h

    g = torch.Generator(device="cuda").manual_seed(9)
    ctx, n_q, heads = [3000, 1500], 400, 32
    cap = max(ctx)
    q = torch.randn((2, n_q, heads, 128), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((2, cap, 128), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((2, cap, 128), generator=g, device="cuda").to(torch.bfloat16)
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    desc = h.make_desc(batch=2, n_heads=heads, n_q=n_q, tile_q=1, k_top=0, window=window)
    res = []
    for kk, vv in ((k, v), (_padded(k.view(torch.int16), ctx, 0x7FC0).view(torch.bfloat16),
                           _padded(v.view(torch.int16), ctx, 0x7FC0).view(torch.bfloat16))):
        o = torch.empty((2, n_q, heads, 128), device="cuda")
        lse = torch.empty((2, n_q, heads), device="cuda")
        h.hs2_swa_attention(desc, q, kk, vv, kk.shape[1] * 128, ctx_t, cap, o, h.HS2_F32, lse)
        res.append((o, lse))
    _say(f"sliding-window attention on a padded cache (window {window})")
    _same(list(res[1]), list(res[0]))
    assert not torch.isnan(res[1][0]).any()
