"""GPU parity of the self-decoder's sliding-window attention (hs2_swa_attention).

Outputs (fp32, and bf16 rounded) are compared with the oracle's fp64
sliding-window attention on the same bf16 inputs (the bf16 output bar) and
the log-sum-exp to 1e-5.  Shapes
cover ragged query counts (not multiples of the 8 queries a workgroup
takes), windows of one key, of 128 and wider than one 64-key tile, windows
that cover the whole context (dense causal attention), padded heads, queries
before the cache start, decode (one query) and a sampled 8,192-query prefill.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_outputs_close
from workloads import WORKLOADS, make_prefill_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _run(inp, w, n_q, window, out="f32"):
    import kv_cache_reuse_hs2_amd as hs2
    from kv_cache_reuse_hs2_amd.torch_api import to_device

    bsz = inp["ctx_len"].shape[0]
    cap = int(inp["capacity"])
    d = hs2.make_desc(batch=bsz, n_heads=w.n_heads, n_q=n_q, tile_q=1, k_top=0, window=window,
                      sm_scale=w.sm_scale)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    o = torch.full((bsz, n_q, w.n_heads, 128), 7.0, dtype=dt, device="cuda")
    lse = torch.full((bsz, n_q, w.n_heads), 7.0, dtype=torch.float32, device="cuda")
    hs2.hs2_swa_attention(d, to_device(inp["q_raw"]), to_device(inp["k_raw"]),
                          to_device(inp["v_raw"]), cap * 128, to_device(inp["ctx_len"]), cap, o,
                          hs2.HS2_F32 if out == "f32" else hs2.HS2_BF16, lse)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


CASES = [
    # name, batch, heads, ctx, cap, n_q, window
    ("w128_ragged", 2, 32, [3000, 1500], 3000, 203, 128),
    ("w1", 1, 32, [900], 900, 77, 1),
    ("w300_multi_tile", 2, 32, [2000, 700], 2000, 150, 300),
    ("dense", 1, 32, [400], 400, 64, 4096),
    ("heads7", 2, 7, [1200, 640], 1200, 96, 128),
    ("before_cache_start", 2, 32, [50, 9], 64, 64, 16),
    ("decode", 4, 32, [5000, 129, 128, 1], 5000, 1, 128),
    ("w129_widest_band", 1, 32, [2000], 2000, 100, 129),
    ("w130_narrowest_tiled", 1, 32, [2000], 2000, 100, 130),
    ("heads1", 2, 1, [700, 333], 700, 70, 128),
]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("name,bsz,heads,ctx,cap,n_q,window", CASES, ids=[c[0] for c in CASES])
def test_swa_matches_oracle(hs2, name, bsz, heads, ctx, cap, n_q, window, out):
    w = WORKLOADS["prefill_bf16_128k_8k"].replace(batch=bsz, n_heads=heads)
    inp = make_prefill_inputs(w, ctx_lens=ctx, n_q=n_q, capacity=cap)
    _say(f"swa {name} ctx={ctx} n_q={n_q} window={window} H={heads} out={out}")
    o, lse = _run(inp, w, n_q, window, out)
    o_ref, lse_ref = oracle.swa_attention(inp["q"], inp["k"], inp["v"], inp["ctx_len"],
                                          window=window, sm_scale=w.sm_scale)
    assert_outputs_close(o, o_ref, "bf16")
    fin = np.isfinite(lse_ref)
    np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=1e-5, atol=1e-5)
    assert np.all(np.isneginf(lse[~fin])) and np.all(o[~fin] == 0)
    if name == "dense":
        o_d, _ = oracle.dense_attention(inp["q"], inp["k"], inp["v"], inp["ctx_len"],
                                        sm_scale=w.sm_scale)
        assert_outputs_close(o, o_d, "bf16")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_swa_full_size_sampled(hs2, out):
    # 8,192 queries at positions 131,072.. of a 139,264-key cache, window 128;
    # the oracle evaluates a seeded sample of queries, each alone (one query
    # whose context ends at its own position).
    w = WORKLOADS["prefill_bf16_128k_8k"]
    inp = make_prefill_inputs(w)
    _say(f"swa full size n_q={w.n_q} ctx={w.ctx_len} out={out}")
    o, lse = _run(inp, w, w.n_q, 128, out)
    assert np.all(np.isfinite(o))
    rng = np.random.default_rng(70)
    sample = np.concatenate([[0, 1, 7, 8, w.n_q - 1], rng.choice(w.n_q, 27, replace=False)])
    for i in sample:
        P = w.ctx_len - w.n_q + int(i)
        o_ref, lse_ref = oracle.swa_attention(inp["q"][:, i:i + 1], inp["k"], inp["v"],
                                              np.array([P + 1]), window=128,
                                              sm_scale=w.sm_scale)
        assert_outputs_close(o[:, i:i + 1], o_ref, "bf16")
        np.testing.assert_allclose(lse[:, i:i + 1], lse_ref, rtol=1e-5, atol=1e-5)
