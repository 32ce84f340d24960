"""The allocation-free decode step against hs2_decode_step, through the C ABI.

hs2_decode_step_noalloc runs the same kernels with its workspace in the
library's device array, so its outputs must equal hs2_decode_step's (with a
caller workspace) bit for bit.  Two calls in a row, the second on a smaller
problem, so the second finds the array as the first left it.
"""

import sys

import numpy as np
import pytest
import torch

from workloads import WORKLOADS, make_decode_inputs

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 32 << 20


def _say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _outputs(buf):
    return [t.clone() for t in (buf.scores, buf.top_idx, buf.top_cnt, buf.o, buf.lse,
                                buf.lse_full)]


def _compare(hs2, wname, over, ctx):
    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_fused_step

    w = WORKLOADS[wname].replace(**over)
    inp = make_decode_inputs(w, ctx_lens=ctx, capacity=max(ctx))
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    assert hs2.hs2_workspace_size(buf.desc, buf.cap) <= SCRATCH_BYTES
    _say(f"no-alloc step {wname} ctx={ctx} dtype={w.dtype}")
    run_fused_step(buf)
    torch.cuda.synchronize()
    ref = _outputs(buf)
    for t in (buf.scores, buf.top_idx, buf.top_cnt, buf.o, buf.lse, buf.lse_full):
        t.fill_(7)
    hs2.hs2_decode_step_noalloc(buf.desc, buf.q, None, buf.k, buf.v, buf.kv_stride, buf.ctx_len,
                                buf.cap, buf.scores, buf.lse_full, buf.top_idx, buf.top_cnt,
                                buf.o, buf.lse)
    torch.cuda.synchronize()
    got = _outputs(buf)
    for b, n in enumerate(ctx):  # scores past a sequence's context are not written
        assert torch.equal(ref[0][b, :, :n], got[0][b, :, :n])
    for a, g in zip(ref[1:], got[1:]):
        assert torch.equal(a, g)


def test_noalloc_step_equals_workspace_step(hs2):
    # A larger problem, then a smaller one on the array it left behind.
    _compare(hs2, "decode_bf16_256k_b4", dict(batch=4), [65536, 40000, 9001, 1153])
    _compare(hs2, "decode_bf16_64k_b16", dict(batch=2, n_heads=7), [9000, 300])
    _compare(hs2, "decode_fp8_256k_b4", dict(batch=2), [20000, 4097])


def test_noalloc_step_rejects_an_oversized_workspace(hs2):
    from kv_cache_reuse_hs2_amd import HS2_EWORKSPACE, HS2Error, make_desc

    d = make_desc(batch=16, n_heads=32)
    cap = 262144
    assert hs2.hs2_workspace_size(d, cap) > SCRATCH_BYTES
    dummy = torch.zeros(64, dtype=torch.float32, device="cuda")
    with pytest.raises(HS2Error) as err:
        hs2.hs2_decode_step_noalloc(d, dummy, None, dummy, dummy, cap * 128, dummy, cap, dummy,
                                    None, dummy, dummy, dummy)
    assert err.value.status == HS2_EWORKSPACE
    np.testing.assert_array_equal(dummy.cpu().numpy(), 0)  # nothing was written
