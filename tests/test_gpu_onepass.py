"""GPU parity of the one-pass decode scoring in the cases that only it has.

The one-pass kernel keeps each workgroup's last logit tiles on chip (as the
terms 2^(x - m) of the running per-head sums, m a reference maximum) and reads
the rest of its keys again after the grid barrier.  A wave whose reference has
to move after it has kept tiles (a logit more than 64 binades above it) reads
all its keys again instead.  These tests plant keys that force such moves at
known places of the launch plan, run shapes that keep tiles in LDS and read
blocks again, reuse one workspace for several batch sizes (the barrier words
sit at fixed places), and take the two-pass path of batches larger than the
GPU's compute unit count.  Bars as in the other decode tests: scores
element-wise 1e-4 relative (and 1e-5 relative L2), selection from GPU scores
only at near-ties, sparse output max abs 2e-2 and relative L2 5e-3.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_outputs_close, assert_scores_close, assert_selection_near_ties
from workloads import WORKLOADS, bf16_bits, bf16_bits_to_f32, make_decode_inputs

pytestmark = pytest.mark.gpu

REG_TILES, LDS_TILES, WAVES = 20, 9, 4  # bf16 kernel's kept tiles per wave


def _say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _plan(batch, cap):
    """Workgroups per sequence and keys per workgroup of the one-pass launch."""
    n_cu = min(torch.cuda.get_device_properties(0).multi_processor_count, 256)
    per_seq = n_cu // batch
    units = (cap + 255) // 256
    n = max(1, min(per_seq, units))
    return n, -(-units // n) * 256


def _key(nwg, wg, wave, block, offset):
    """Key index of `offset` within local block `block` of `wave` in workgroup
    `wg` of a sequence's nwg: workgroup wg takes the 32-key blocks wg,
    wg + nwg, wg + 2 nwg, ..., its waves in turn."""
    return 32 * ((block * WAVES + wave) * nwg + wg) + offset


def _plant(inp, places, size=100.0):
    """Set k[b, j] = size * unit(q[b, head 0]) (bf16) at each (b, j) of places."""
    k = inp["k"].copy()
    for b, j in places:
        u = inp["q"][b, 0, 0].astype(np.float64)
        k[b, j] = (size * u / np.linalg.norm(u)).astype(np.float32)
    bits = bf16_bits(k)
    inp = dict(inp, k=bf16_bits_to_f32(bits), k_raw=bits)
    # The planted logits of head 0 are far above every other logit of head 0,
    # so the wave that meets one must move its reference.
    c2 = 1.4426950408889634 / np.sqrt(128.0)
    for b, j in places:
        q0 = inp["q"][b, 0, 0].astype(np.float64)
        x = c2 * (inp["k"][b].astype(np.float64) @ q0)
        others = np.delete(x, [jj for bb, jj in places if bb == b])
        assert x[j] - others.max() > 64.0
    return inp


def _check_step(hs2, w, inp, ctx):
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_fused_step, run_scores

    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    run_scores(buf)
    torch.cuda.synchronize()
    ref, _, _ = oracle.full_attn_scores(inp["q"], inp["k"], inp["ctx_len"], tile_q=1,
                                        sm_scale=w.sm_scale)
    scores = buf.scores.cpu().numpy()
    assert_scores_close(scores, ref, ctx)
    run_fused_step(buf)
    torch.cuda.synchronize()
    assert np.array_equal(buf.scores.cpu().numpy()[:, :, :min(ctx)], scores[:, :, :min(ctx)])
    top, cnt = oracle.select_topk_window(ref, inp["ctx_len"], n_q=1, tile_q=1, k_top=w.k_top,
                                         window=w.window)
    tg, cg = buf.top_idx.cpu().numpy(), buf.top_cnt.cpu().numpy()
    assert_selection_near_ties(tg, cg, top, cnt, ref, inp["ctx_len"], n_q=1, tile_q=1,
                               window=w.window)
    o_ref, _ = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["ctx_len"], tg, cg,
                                       tile_q=1, window=w.window, sm_scale=w.sm_scale)
    assert_outputs_close(buf.o.cpu().numpy(), o_ref, w.dtype)
    return buf


def test_late_reference_move_register_tiles(hs2):
    # 2 x 9,000 keys: 36 workgroups of 256 keys per sequence, two blocks per
    # wave, both kept in registers.  Each planted key is in a wave's second
    # block, met after the wave kept its first.
    w = WORKLOADS["decode_bf16_64k_b16"].replace(batch=2)
    ctx = [9000, 5000]
    nwg, chunk = _plan(2, 9000)
    assert (nwg, chunk) == (36, 256)
    places = [(0, _key(nwg, 0, 1, 1, 1)), (1, _key(nwg, 9, 0, 1, 30))]
    assert all(j < ctx[b] for b, j in places)
    inp = _plant(make_decode_inputs(w, ctx_lens=ctx, capacity=max(ctx)), places)
    _say(f"late move, register tiles, places={places}")
    _check_step(hs2, w, inp, ctx)


def test_late_reference_move_lds_tiles(hs2):
    # 16 x 45,056 keys: 2,816 keys per workgroup, 22 blocks per wave; blocks 0
    # and 1 are kept in LDS, 2..21 in registers.  Planted keys in register
    # blocks (after LDS tiles were kept) and in an LDS block (after block 0).
    w = WORKLOADS["decode_bf16_64k_b16"].replace(batch=16)
    cap = 45056
    ctx = [cap] * 15 + [30001]
    nwg, chunk = _plan(16, cap)
    assert (nwg, chunk) == (16, 2816)
    places = [(0, _key(nwg, 3, 2, 5, 7)), (5, _key(nwg, 0, 0, 1, 0)),
              (15, _key(nwg, 9, 1, 14, 31))]
    assert all(j < ctx[b] for b, j in places)
    inp = _plant(make_decode_inputs(w, ctx_lens=ctx, capacity=cap), places)
    _say(f"late move, LDS tiles, places={places}")
    _check_step(hs2, w, inp, ctx)


def test_late_reference_move_with_reread_blocks(hs2):
    # 4 x 262,144 keys: 4,096 keys per workgroup, 32 blocks per wave: blocks
    # 0..2 read again, 3..11 kept in LDS, 12..31 in registers.  Planted keys
    # in an LDS block and in a register block (late moves: those waves read
    # all 32 blocks again), and in block 1 (a move before anything is kept: no
    # fallback).
    w = WORKLOADS["decode_bf16_256k_b4"]
    cap = w.ctx_len
    ctx = [cap, cap, cap - 5000, 140000]
    nwg, chunk = _plan(4, cap)
    assert (nwg, chunk) == (64, 4096)
    places = [(0, _key(nwg, 10, 0, 10, 3)), (1, _key(nwg, 20, 3, 1, 9)),
              (3, _key(nwg, 33, 0, 16, 0))]
    assert all(j < ctx[b] for b, j in places)
    inp = _plant(make_decode_inputs(w, ctx_lens=ctx, capacity=cap), places)
    _say(f"late move with read-again blocks, places={places}")
    _check_step(hs2, w, inp, ctx)


def test_late_reference_move_fp8(hs2):
    import torch as _t  # noqa: F401

    from workloads.generators import e4m3_codes

    w = WORKLOADS["decode_fp8_256k_b4"].replace(batch=2)
    ctx = [9000, 5000]
    nwg, chunk = _plan(2, 9000)
    places = [(0, _key(nwg, 0, 1, 1, 1)), (1, _key(nwg, 9, 0, 1, 30))]
    assert all(j < ctx[b] for b, j in places)
    base = make_decode_inputs(w.replace(dtype="bf16"), ctx_lens=ctx, capacity=max(ctx))
    planted = _plant(base, places)
    k_raw, k_scale = e4m3_codes(planted["k"])
    v_raw, v_scale = e4m3_codes(planted["v"])
    inp = dict(planted, k_raw=k_raw, v_raw=v_raw, k_scale=k_scale, v_scale=v_scale,
               k=oracle.dequant_kv(k_raw, k_scale), v=oracle.dequant_kv(v_raw, v_scale))
    _say(f"late move, E4M3 cache, places={places}")
    _check_step(hs2, w, inp, ctx)


def test_workspace_reused_across_batch_sizes(hs2):
    # One workspace (sized for the largest call) serves calls of 4, 2 and 4
    # sequences in turn; the barrier words keep their places.
    from kv_cache_reuse_hs2_amd import hs2_decode_step, hs2_workspace_size, make_desc
    from kv_cache_reuse_hs2_amd.torch_api import to_device

    w = WORKLOADS["decode_bf16_256k_b4"]
    cap = 20000
    inp = make_decode_inputs(w, ctx_lens=[20000, 17000, 9001, 4000], capacity=cap)
    ref, _, _ = oracle.full_attn_scores(inp["q"], inp["k"], inp["ctx_len"], tile_q=1,
                                        sm_scale=w.sm_scale)
    size = max(hs2_workspace_size(make_desc(batch=bb, n_heads=w.n_heads), cap) for bb in (2, 4))
    ws = torch.full((size,), 0xA5, dtype=torch.uint8, device="cuda")  # not zero-filled
    q, k, v = (to_device(inp[x]) for x in ("q_raw", "k_raw", "v_raw"))
    ctx = to_device(inp["ctx_len"])
    for bsz in (4, 2, 4, 2):
        _say(f"workspace reuse: batch {bsz}")
        d = make_desc(batch=bsz, n_heads=w.n_heads)
        scores = torch.zeros((bsz, 1, cap), dtype=torch.float32, device="cuda")
        ti = torch.empty((bsz, 1, w.k_top), dtype=torch.int32, device="cuda")
        tc = torch.empty((bsz, 1), dtype=torch.int32, device="cuda")
        o = torch.empty((bsz, 1, w.n_heads, 128), dtype=torch.float32, device="cuda")
        hs2_decode_step(d, q[:bsz], None, k[:bsz], v[:bsz], cap * 128, ctx[:bsz], cap, scores,
                        None, ti, tc, o, None, ws)
        torch.cuda.synchronize()
        assert_scores_close(scores.cpu().numpy(), ref[:bsz], inp["ctx_len"][:bsz])


def test_two_pass_path_beyond_the_compute_units(hs2):
    # More sequences than compute units: the two-pass kernels, same results.
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_fused_step, run_step

    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    bsz = n_cu + 4
    w = WORKLOADS["decode_bf16_64k_b16"].replace(batch=bsz, n_heads=8)
    rng = np.random.default_rng(77)
    ctx = rng.integers(1, 1500, size=bsz).tolist()
    ctx[0] = 1500
    inp = make_decode_inputs(w, ctx_lens=ctx, capacity=1500)
    _say(f"two-pass path, batch {bsz}")
    _check_step(hs2, w, inp, ctx)
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    run_step(buf)
    torch.cuda.synchronize()
    three = [t.clone() for t in (buf.top_idx, buf.top_cnt, buf.o)]
    run_fused_step(buf)
    torch.cuda.synchronize()
    for a, b in zip(three, (buf.top_idx, buf.top_cnt, buf.o)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("extra,cap", [(0, 1500), (1, 1500), (1, 8192), (None, 1500)],
                         ids=["two_wg_per_seq", "one_wg_per_seq", "one_wg_long", "batch_eq_cus"])
def test_few_workgroups_per_sequence(hs2, extra, cap):
    # Batches near the compute unit count: two workgroups per sequence, one
    # (each workgroup then takes the whole sequence: at 8,192 keys its waves
    # keep 29 of their 64 blocks and read the other 35 again), and exactly one
    # sequence per compute unit.  Same bars; the single call equals the three.
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_fused_step, run_step

    n_cu = min(torch.cuda.get_device_properties(0).multi_processor_count, 256)
    bsz = n_cu if extra is None else n_cu // 2 + extra
    nwg, chunk = _plan(bsz, cap)
    assert nwg == (2 if extra == 0 else 1) and chunk >= cap // nwg
    w = WORKLOADS["decode_bf16_64k_b16"].replace(batch=bsz, n_heads=8)
    rng = np.random.default_rng(1000 + bsz + cap)
    ctx = rng.integers(1, cap + 1, size=bsz).tolist()
    ctx[0] = cap
    inp = make_decode_inputs(w, ctx_lens=ctx, capacity=cap)
    _say(f"batch {bsz}, {nwg} workgroup(s) per sequence, capacity {cap}")
    _check_step(hs2, w, inp, ctx)
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    run_step(buf)
    torch.cuda.synchronize()
    three = [t.clone() for t in (buf.top_idx, buf.top_cnt, buf.o)]
    run_fused_step(buf)
    torch.cuda.synchronize()
    for a, b in zip(three, (buf.top_idx, buf.top_cnt, buf.o)):
        assert torch.equal(a, b)
