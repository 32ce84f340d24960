"""Shared helpers of the GPU parity tests (not a test module).

Tolerances (the bar each GPU test asserts):
* importance scores: element-wise |gpu - oracle| <= 1e-4 * |oracle| + 1e-30
  and, per sequence and tile, relative L2 error <= 1e-5 (both sides compute
  in fp32 or better on identical stored inputs);
* selection fed the oracle's fp32 scores: bit-exact;
* selection from GPU scores: every index in the symmetric difference with the
  oracle's selection is a near-tie, |I_or[j] - tau| <= 1e-4 * tau, tau being
  the oracle's k-th pool score;
* sparse outputs: max |gpu - oracle| <= 1e-4 for fp32 storage; for bf16
  and E4M3 storage (the E4M3 kernels widen the bytes to bf16 exactly and
  then compute as the bf16 ones) max abs <= 2e-2 and relative L2 <= 5e-3;
* bridge: within one bfloat16 ulp of the oracle's correctly rounded value,
  relative L2 <= 5e-3.
"""

from __future__ import annotations

import numpy as np

import oracle

SCORE_RTOL = 1e-4
SCORE_ATOL = 1e-30
SCORE_REL_L2 = 1e-5


def assert_scores_close(gpu: np.ndarray, ref: np.ndarray, ctx_len) -> None:
    for b, n in enumerate(ctx_len):
        g = gpu[b, :, :n].astype(np.float64)
        r = ref[b, :, :n].astype(np.float64)
        err = np.abs(g - r)
        bad = err > SCORE_RTOL * np.abs(r) + SCORE_ATOL
        assert not bad.any(), (
            f"seq {b}: {bad.sum()} scores off, worst rel "
            f"{(err / np.maximum(np.abs(r), 1e-30)).max():.3e}")
        for t in range(r.shape[0]):
            den = np.linalg.norm(r[t])
            if den > 0:
                rel = np.linalg.norm(g[t] - r[t]) / den
                assert rel <= SCORE_REL_L2, f"seq {b} tile {t}: relative L2 {rel:.3e}"


def assert_outputs_close(gpu: np.ndarray, ref: np.ndarray, dtype: str) -> None:
    gpu = gpu.astype(np.float64)
    err = np.abs(gpu - ref)
    if dtype == "f32":
        assert err.max() <= 1e-4, f"max abs {err.max():.3e}"
    else:
        assert err.max() <= 2e-2, f"max abs {err.max():.3e}"
        den = np.linalg.norm(ref)
        rel = np.linalg.norm(gpu - ref) / den if den > 0 else np.linalg.norm(gpu)
        assert rel <= 5e-3, f"rel L2 {rel:.3e}"


def assert_selection_near_ties(top_gpu, cnt_gpu, top_or, cnt_or, scores_or, ctx_len, *, n_q,
                               tile_q, window) -> int:
    """End-to-end selection check; returns the number of near-tie swaps."""
    swaps = 0
    for b in range(top_or.shape[0]):
        pos = oracle.query_positions(int(ctx_len[b]), n_q)
        for t in range(top_or.shape[1]):
            assert cnt_gpu[b, t] == cnt_or[b, t]
            c = int(cnt_or[b, t])
            g = top_gpu[b, t, :c]
            assert np.all(np.diff(g) > 0), "not ascending"
            pe = oracle.pool_end(pos[t * tile_q], window)
            assert c == 0 or (g.min() >= 0 and g.max() < pe)
            assert np.all(top_gpu[b, t, c:] == -1)
            o = top_or[b, t, :c]
            diff = np.setxor1d(g, o)
            if diff.size:
                imp = scores_or[b, t, :pe].astype(np.float64)
                tau = np.sort(imp)[::-1][c - 1]
                assert np.all(np.abs(imp[diff] - tau) <= 1e-4 * tau), "selection differs beyond near-ties"
                swaps += diff.size // 2
    return swaps


def assert_prefill_out_close(got, o_ref, o_abs, vmax, what):
    """Prefill o_full against the oracle: 1e-4 * max|v| for the fp32 work plus
    2^-8 * sum_j p_j |v_j| for p's bf16 rounding, per output; and the bf16
    path's bar (max abs 2e-2, relative L2 5e-3)."""
    err = np.abs(got - o_ref)
    bound = 1e-4 * vmax + 2.0 ** -8 * o_abs
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"{what}: o_full error {worst:.3f} of its bound (max abs {err.max():.3e})"
    assert err.max() <= 2e-2, f"{what}: o_full max abs {err.max():.3e}"
    rel = float(np.linalg.norm(got - o_ref) / max(np.linalg.norm(o_ref), 1e-30))
    assert rel <= 5e-3, f"{what}: o_full relative L2 {rel:.3e}"
    print(f"[gpu] {what}: max abs {err.max():.3e}, {100 * worst:.1f}% of the bound, rel L2 {rel:.2e}", flush=True)
