"""Several sparse layers sharing one selection (one gather for all layers).

Each layer's output must equal a separate hs2_sparse_attn_gather call with
that layer's query, bit for bit, and the oracle's sparse attention over the
same selection within the bf16 bar.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_outputs_close
from workloads import WORKLOADS, make_decode_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("n_layers,ctx", [(1, [5000, 3000, 1200, 1]), (3, [5000, 3000, 1200, 0]),
                                          (8, [2000, 2000, 1300, 100])])
def test_layers_equal_separate_calls_and_oracle(hs2, n_layers, ctx):
    from kv_cache_reuse_hs2_amd.torch_api import (make_buffers, run_sparse, run_sparse_layers,
                                                  run_step, to_device)

    w = WORKLOADS["decode_bf16_256k_b4"]
    cap = max(ctx)
    inp = make_decode_inputs(w, ctx_lens=ctx, capacity=cap)
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype="bf16")
    _say(f"layers={n_layers} ctx={ctx}")
    run_step(buf)
    qs = [inp] + [make_decode_inputs(w, seed=w.seed + 100 + l, ctx_lens=ctx, capacity=cap)
                  for l in range(1, n_layers)]
    q_layers = to_device(np.stack([x["q_raw"] for x in qs]))
    o_l, lse_l = run_sparse_layers(buf, q_layers)
    torch.cuda.synchronize()
    tg, cg = buf.top_idx.cpu().numpy(), buf.top_cnt.cpu().numpy()
    for l in range(n_layers):
        run_sparse(buf, q=q_layers[l])
        torch.cuda.synchronize()
        assert torch.equal(buf.o, o_l[l]) and torch.equal(buf.lse, lse_l[l]), f"layer {l}"
        o_ref, lse_ref = oracle.sparse_attention(qs[l]["q"], inp["k"], inp["v"], inp["ctx_len"],
                                                 tg, cg, tile_q=1, window=w.window,
                                                 sm_scale=w.sm_scale)
        assert_outputs_close(o_l[l].cpu().numpy(), o_ref, "bf16")
        fin = np.isfinite(lse_ref)
        np.testing.assert_allclose(lse_l[l].cpu().numpy()[fin], lse_ref[fin], rtol=1e-5, atol=1e-5)
        assert np.all(np.isneginf(lse_l[l].cpu().numpy()[~fin]))
