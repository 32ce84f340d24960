"""Decode-step benchmark of the HySparse2 KV Reuse hot path on one MI355X.

One step = one decode step of every sequence of the batch through the whole
hot path: full-layer scoring (hs2_full_attn_scores), top-1024 + window-128
selection (hs2_select_topk_window) and the sparse layer
(hs2_sparse_attn_gather), on the 256k-context workload: batch 4, 32 query
heads sharing one bf16 K/V head of dim 128, 262,144 cached keys per sequence,
keys drawn as N(0,1) background plus 0.1% clustered high-similarity keys.
Inputs are synthetic, seeded and resident in HBM before timing starts.

Prints one JSON line.  value = decoded tokens/s = batch * steps / time, the
steps cycling over four distinct K/V caches (as a model's full layers would),
so that no step finds its K left in the memory-side cache by the step before.
Also reported: the step's algorithmic HBM GB/s (K read once, scores written
and read once, 1,152 gathered K and V rows per sequence), a roofline entry
for the dominant unit of work (the scoring call, timed with HIP events on
its own stream), one sequence of the last step checked against the oracle,
and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
WORKLOAD = "decode_bf16_256k_b4"
GRAPH_STEPS = 10  # decode steps per captured HIP graph (extras)
GRAPH_ROUNDS = 3  # rounds over the four caches per captured HIP graph (headline)
# The headline scoring call's kernel (bf16 K, no selector histogram).
SCORE_KERNEL = "score_onepass<false, false, 20>"
# The sources of the headline scoring kernel: its measured traffic is used only
# while these are unchanged.
TRAFFIC_SOURCES = ("score_onepass.hip", "score_common.h", "select_core.h", "hs2_internal.h", "layout.h")
MIB = 1 << 20


def algorithmic_bytes(w) -> dict:
    """Bytes a decode step must move at minimum (K/V rows of 256 B in bf16,
    128 B in E4M3)."""
    n, b = w.ctx_len, w.batch
    row = w.head_dim * {"f32": 4, "bf16": 2, "fp8": 1}[w.dtype]
    k_stream = b * n * row                      # every key read once
    scores = b * n * 4                          # importance written once ...
    pool = b * max(0, n - w.window) * 4         # ... and the pool read once by the selector
    sel = min(n, w.k_top + w.window)
    gather = b * sel * 2 * row                  # K and V rows of the selection
    q_o = b * w.n_heads * w.head_dim * (2 + 4 + 2)
    return dict(k_stream=k_stream, scores_write=scores, scores_read=pool, gather=gather,
                q_out=q_o, step=k_stream + scores + pool + gather + q_o,
                scoring_call=k_stream + scores)


def time_events(fn, steps: int, warmup: int) -> float:
    """Average milliseconds of fn() over `steps` runs, HIP events on the
    current stream, after `warmup` untimed runs."""
    import torch

    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_graphs(fn, steps: int, warmup: int) -> float:
    """Average milliseconds of fn() replayed from HIP graphs of GRAPH_STEPS
    consecutive calls (as the headline step), HIP events around exactly
    `steps` calls."""
    import torch

    stream = torch.cuda.current_stream()
    per = min(GRAPH_STEPS, steps)
    graphs = {}
    for n in {per, 1}:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            fn()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        graphs[n] = g
    torch.cuda.synchronize()
    for _ in range(warmup):
        graphs[1].replay()
    torch.cuda.synchronize()
    plan = [graphs[per]] * (steps // per) + [graphs[1]] * (steps % per)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for g in plan:
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def sparse_layer_measurements(steps: int, warmup: int) -> dict:
    """S sparse layers after the full layer, sharing its selection: the decode
    step (scoring, selection, first sparse layer) plus S-1 further layers in
    one gather (hs2_sparse_attn_gather_layers), against S-1 separate
    hs2_sparse_attn_gather calls."""
    import numpy as np
    import torch

    from kv_cache_reuse_hs2_amd.torch_api import (make_buffers, run_fused_step, run_sparse,
                                                  run_sparse_layers, to_device)
    from workloads import WORKLOADS, make_decode_inputs

    w = WORKLOADS[WORKLOAD]
    inp = make_decode_inputs(w)
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    rng = np.random.Generator(np.random.PCG64(w.seed + 7))
    out = {}
    for n_sparse in (1, 2, 4, 8):
        extra = n_sparse - 1
        if extra:
            q = rng.standard_normal((extra,) + inp["q_raw"].shape, dtype=np.float32)
            q_layers = to_device(q).to(torch.bfloat16).view(torch.int16)
            step = lambda: (run_fused_step(buf), run_sparse_layers(buf, q_layers))  # noqa: E731
            sep = lambda: (run_fused_step(buf),  # noqa: E731
                           [run_sparse(buf, q=q_layers[i]) for i in range(extra)])
        else:
            step = sep = lambda: run_fused_step(buf)  # noqa: E731
        ms = time_graphs(step, steps, warmup)
        ms_sep = time_graphs(sep, steps, warmup)
        out[f"sparse_layers_{n_sparse}"] = {
            "ms_per_step": round(ms, 5), "tokens_per_s": round(w.batch / (ms * 1e-3), 1),
            "ms_per_step_separate_calls": round(ms_sep, 5)}
    return out


def block_measurements(steps: int, warmup: int) -> dict:
    """Token-level against block-level (64-token blocks) selection at the same
    budget on the headline workload: the single-call step of each, and the
    selection and sparse calls alone (HIP events per call)."""
    import torch

    from kv_cache_reuse_hs2_amd.torch_api import (make_buffers, run_fused_step,
                                                  run_fused_step_blocks, run_scores,
                                                  run_select, run_select_blocks, run_sparse)
    from workloads import WORKLOADS, make_decode_inputs

    w = WORKLOADS[WORKLOAD]
    buf = make_buffers(make_decode_inputs(w), n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    out = {"block": 64}
    out["step_ms_token"] = round(time_graphs(lambda: run_fused_step(buf), steps, warmup), 5)
    out["step_ms_block"] = round(time_graphs(lambda: run_fused_step_blocks(buf, 64), steps,
                                             warmup), 5)
    run_scores(buf)
    out["select_ms_token"] = round(time_events(lambda: run_select(buf), steps, warmup), 5)
    run_select(buf)
    out["sparse_ms_token"] = round(time_events(lambda: run_sparse(buf), steps, warmup), 5)
    out["select_ms_block"] = round(time_events(lambda: run_select_blocks(buf, 64), steps,
                                               warmup), 5)
    run_select_blocks(buf, 64)
    out["sparse_ms_block"] = round(time_events(lambda: run_sparse(buf), steps, warmup), 5)
    torch.cuda.synchronize()
    out["selected_rows_block"] = int(buf.top_cnt.sum().item())
    out["tokens_per_s_block"] = round(w.batch / (out["step_ms_block"] * 1e-3), 1)
    return out


def swa_measurements(steps: int, warmup: int) -> dict:
    """The self-decoder's sliding-window attention (hs2_swa_attention) over the
    chunked-prefill shape: 8,192 queries at the end of a 139,264-key cache,
    32 heads, window 128."""
    import torch

    import kv_cache_reuse_hs2_amd as hs2
    from kv_cache_reuse_hs2_amd.torch_api import to_device
    from workloads import WORKLOADS, make_prefill_inputs

    w = WORKLOADS["prefill_bf16_128k_8k"]
    inp = make_prefill_inputs(w)
    window = 128
    d = hs2.make_desc(batch=1, n_heads=w.n_heads, n_q=w.n_q, tile_q=1, k_top=0, window=window,
                      sm_scale=w.sm_scale)
    q, k, v = (to_device(inp[x]) for x in ("q_raw", "k_raw", "v_raw"))
    ctx = to_device(inp["ctx_len"])
    lse = torch.empty((1, w.n_q, w.n_heads), dtype=torch.float32, device="cuda")
    cap = int(inp["capacity"])
    nq, hd = w.n_q, w.head_dim
    flop = 4.0 * w.n_heads * hd * nq * window    # QK^T and PV over each query's window
    out = {"window": window, "algorithmic_flop": flop}
    for name, dt, code, ob in (("bf16_out", torch.bfloat16, hs2.HS2_BF16, 2),
                               ("f32_out", torch.float32, hs2.HS2_F32, 4)):
        o = torch.empty((1, nq, w.n_heads, hd), dtype=dt, device="cuda")
        ms = time_events(lambda: hs2.hs2_swa_attention(d, q, k, v, cap * hd, ctx, cap, o, code,
                                                       lse), steps, warmup)
        byts = nq * w.n_heads * hd * (2 + ob) + nq * w.n_heads * 4 + (nq + window - 1) * hd * 4
        out[name] = {"ms": round(ms, 5), "queries_per_s": round(nq / (ms * 1e-3), 1),
                     "hbm_GBps": round(byts / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "achieved_TFLOPs": round(flop / (ms * 1e-3) / 1e12, 1),
                     "algorithmic_bytes": int(byts)}
        del o
    # A wide window takes the streaming (tiled) kernel.
    wide = 1024
    dw = hs2.make_desc(batch=1, n_heads=w.n_heads, n_q=w.n_q, tile_q=1, k_top=0, window=wide,
                       sm_scale=w.sm_scale)
    o = torch.empty((1, nq, w.n_heads, hd), dtype=torch.bfloat16, device="cuda")
    ms = time_events(lambda: hs2.hs2_swa_attention(dw, q, k, v, cap * hd, ctx, cap, o,
                                                   hs2.HS2_BF16, lse), steps, warmup)
    flop_w = 4.0 * w.n_heads * hd * nq * wide
    out["bf16_out_window_1024"] = {"ms": round(ms, 5), "queries_per_s": round(nq / (ms * 1e-3), 1),
                                   "achieved_TFLOPs": round(flop_w / (ms * 1e-3) / 1e12, 1),
                                   "mfma_bf16_frac": round(flop_w / (ms * 1e-3) / 2.5e15, 4),
                                   "kernel": "swa_tiled_bf16 (windows above 129)"}
    del o
    out["note"] = "q read and o written once, the band's K and V rows once"
    return out


def fp8_measurements(steps: int, warmup: int) -> dict:
    """The headline decode step on an FP8 E4M3 K/V cache (same shape, same
    timing method): the step from HIP graphs and the scoring call alone."""
    import numpy as np
    import torch

    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_fused_step, run_scores
    from workloads import WORKLOADS, make_decode_inputs

    w = WORKLOADS["decode_fp8_256k_b4"]
    buf = make_buffers(make_decode_inputs(w), n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    ms = time_graphs(lambda: run_fused_step(buf), steps, warmup)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        run_scores(buf)
    ev = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run_scores(buf)
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    ms_sc = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    ab = algorithmic_bytes(w)
    sc_gbs = ab["scoring_call"] / (ms_sc * 1e-3) / 1e9
    return {"ms_per_step": round(ms, 5), "tokens_per_s": round(w.batch / (ms * 1e-3), 1),
            "step_algorithmic_MiB": round(ab["step"] / MIB, 2),
            "step_hbm_GBps": round(ab["step"] / (ms * 1e-3) / 1e9, 1),
            "scoring_call_ms": round(ms_sc, 5),
            "scoring_call_hbm_GBps": round(sc_gbs, 1),
            "scoring_call_hbm_frac": round(sc_gbs / HBM_PEAK_GBS, 4),
            "note": "K and V as E4M3 bytes with one fp32 scale each, bf16 queries"}


def full_output_measurements(steps: int, warmup: int) -> dict:
    """The full-attention layer itself on the headline shape: the scoring call
    that also writes the layer's own output o_full (K streamed twice, V once),
    timed per call beside the scoring call without it."""
    import numpy as np
    import torch

    from kv_cache_reuse_hs2_amd.torch_api import make_buffers, run_scores, run_scores_full
    from workloads import WORKLOADS, make_decode_inputs

    w = WORKLOADS["decode_bf16_256k_b4"]
    buf = make_buffers(make_decode_inputs(w), n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    o_full = torch.empty((w.batch, w.n_heads, w.head_dim), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    fns = {"scores": lambda: run_scores(buf), "scores_and_o_full": lambda: run_scores_full(buf, o_full)}
    for _ in range(warmup):
        for fn in fns.values():
            fn()
    ev = {k: [] for k in fns}
    for _ in range(steps):
        for name, fn in fns.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev[name].append((e0, e1))
    torch.cuda.synchronize()
    ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}
    row = w.head_dim * 2
    kv_once = 2 * w.batch * w.ctx_len * row + w.batch * w.ctx_len * 4   # K, V, scores
    moved = 3 * w.batch * w.ctx_len * row + w.batch * w.ctx_len * 4     # K twice, V once
    t = ms["scores_and_o_full"] * 1e-3
    return {"scores_us": round(ms["scores"] * 1e3, 2),
            "scores_and_o_full_us": round(ms["scores_and_o_full"] * 1e3, 2),
            "bytes_moved_GBps": round(moved / t / 1e9, 1),
            "bytes_moved_frac": round(moved / t / 1e9 / HBM_PEAK_GBS, 4),
            "kv_once_GBps": round(kv_once / t / 1e9, 1),
            "note": "bytes_moved counts K twice and V once (what the kernels read); kv_once "
                    "counts K and V once, the least a full layer can read"}


def mfma_calibration(steps: int, warmup: int) -> dict:
    """What a library GEMM (torch.matmul in bf16, hipBLASLt) reaches on this
    part, on random and on all-zero operands: a square 8192^3 product, and the
    KV Bridging shape [1,048,576 x 2048] x [2048 x 256] (H times [W_K | W_V])
    that hs2_bridge_kv_packed computes.  A reference for the MFMA-bound
    kernels' fractions, not a part of the path."""
    import torch

    out = {}
    for name, (m, kk, n) in (("square_8192", (8192, 8192, 8192)),
                             ("bridge_shape_1m_x_2048_x_256", (1 << 20, 2048, 256))):
        g = torch.Generator(device="cuda").manual_seed(5)
        a = torch.randn((m, kk), generator=g, device="cuda").to(torch.bfloat16)
        b = torch.randn((kk, n), generator=g, device="cuda").to(torch.bfloat16)
        flop = 2.0 * m * n * kk
        ms = time_events(lambda: torch.matmul(a, b), max(5, steps // 5), 3)
        a.zero_()
        b.zero_()
        ms0 = time_events(lambda: torch.matmul(a, b), max(5, steps // 5), 3)
        out[name] = {"ms": round(ms, 4), "TFLOPs": round(flop / (ms * 1e-3) / 1e12, 1),
                     "mfma_bf16_frac": round(flop / (ms * 1e-3) / 2.5e15, 4),
                     "ms_zero_operands": round(ms0, 4),
                     "TFLOPs_zero_operands": round(flop / (ms0 * 1e-3) / 1e12, 1)}
        del a, b
    out["note"] = ("torch.matmul bf16 (hipBLASLt); the matrix cores' rate depends on the "
                   "operand data, so random and zero operands are both given")
    return out


def extra_measurements(steps: int, warmup: int) -> dict:
    """The other shapes of the method, measured the same way (not the headline):
    batched decode at 64k, chunked prefill of 8,192 queries on a 131,072-token
    cache (bf16 and E4M3 K/V), and KV Bridging of 1,048,576 hidden states followed by a decode step
    over the bridged 1M-token cache."""
    import torch

    import kv_cache_reuse_hs2_amd as hs2
    from kv_cache_reuse_hs2_amd.torch_api import (make_buffers, run_fused_step, run_scores,
                                                  run_scores_full)
    from workloads import WORKLOADS, make_decode_inputs, make_prefill_inputs

    out = {}
    # The small fp32 case (one sequence of 4,096 keys, 16 heads): latency only.
    w = WORKLOADS["decode_f32_4k"]
    buf = make_buffers(make_decode_inputs(w), n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    ms = time_events(lambda: run_fused_step(buf), steps, warmup)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_fused_step(buf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run_fused_step(buf)
    ms_g = time_events(g.replay, steps, warmup)
    out[w.name] = {"us_per_step_eager": round(ms * 1e3, 2),
                   "us_per_step_graph": round(ms_g * 1e3, 2),
                   "note": "fp32 cache, VALU kernels; a latency figure, no roofline claim "
                           "(eager: launch-bound from Python; graph: one-step replays)"}
    del buf, g
    # Batched decode, 16 x 65,536 keys.
    w = WORKLOADS["decode_bf16_64k_b16"]
    buf = make_buffers(make_decode_inputs(w), n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    ms = time_events(lambda: run_fused_step(buf), steps, warmup)
    ab = algorithmic_bytes(w)
    out[w.name] = {"ms_per_step": round(ms, 5), "tokens_per_s": round(w.batch / (ms * 1e-3), 1),
                   "step_hbm_GBps": round(ab["step"] / (ms * 1e-3) / 1e9, 1)}
    del buf
    # Chunked prefill: 8,192 queries, 139,264 keys, tiles of 64.
    w = WORKLOADS["prefill_bf16_128k_8k"]
    inp = make_prefill_inputs(w)
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype, n_q=w.n_q, tile_q=w.tile_q)
    ms = time_events(lambda: run_fused_step(buf), max(2, steps // 10), 2)
    pos = [w.ctx_len - w.n_q + i for i in range(w.n_q)]
    qk_flop = 2.0 * w.n_heads * w.head_dim * sum(p + 1 for p in pos)   # causal QK^T, once
    sel = w.k_top + w.window
    sparse_flop = 2.0 * 2.0 * w.n_heads * w.head_dim * w.n_q * sel      # QK^T + PV over 1,152 keys
    alg = qk_flop + sparse_flop
    out[w.name] = {"ms_per_step": round(ms, 4), "queries_per_s": round(w.n_q / (ms * 1e-3), 1),
                   "algorithmic_TFLOP": round(alg / 1e12, 3),
                   "achieved_TFLOPs": round(alg / (ms * 1e-3) / 1e12, 1),
                   "mfma_bf16_frac": round(alg / (ms * 1e-3) / 2.5e15, 4),
                   "note": "algorithmic FLOPs count the causal QK^T once plus the sparse "
                           "QK^T+PV; the recompute pass is overhead"}
    # The full layer's own output on the same shape: scoring alone, then
    # scoring with o_full (one more pass over K and V).
    o_full = torch.empty((1, w.n_q, w.n_heads, w.head_dim), dtype=torch.float32, device="cuda")
    ms_s = time_events(lambda: run_scores(buf), max(2, steps // 10), 2)
    ms_f = time_events(lambda: run_scores_full(buf, o_full), max(2, steps // 10), 2)
    att_flop = 2.0 * qk_flop   # causal QK^T and P.V, once each
    out[w.name]["full_layer"] = {
        "scores_ms": round(ms_s, 4), "scores_and_o_full_ms": round(ms_f, 4),
        "o_full_pass_ms": round(ms_f - ms_s, 4),
        "attention_TFLOPs": round(att_flop / (ms_f * 1e-3) / 1e12, 1),
        "o_full_pass_TFLOPs": round(att_flop / ((ms_f - ms_s) * 1e-3) / 1e12, 1),
        "note": "attention FLOPs count the causal QK^T and P.V once each; the output pass "
                "recomputes QK^T and multiplies P rounded to bf16"}
    del buf, inp, o_full
    # The same prefill on an E4M3 K/V cache (one scale per cache).
    w8 = WORKLOADS["prefill_fp8_128k_8k"]
    inp = make_prefill_inputs(w8)
    buf = make_buffers(inp, n_heads=w8.n_heads, k_top=w8.k_top, window=w8.window,
                       sm_scale=w8.sm_scale, dtype="fp8", n_q=w8.n_q, tile_q=w8.tile_q)
    ms8 = time_events(lambda: run_fused_step(buf), max(2, steps // 10), 2)
    ms8_s = time_events(lambda: run_scores(buf), max(2, steps // 10), 2)
    o_full = torch.empty((1, w8.n_q, w8.n_heads, w8.head_dim), dtype=torch.float32, device="cuda")
    ms8_f = time_events(lambda: run_scores_full(buf, o_full), max(2, steps // 10), 2)
    out[w8.name] = {"ms_per_step": round(ms8, 4), "queries_per_s": round(w8.n_q / (ms8 * 1e-3), 1),
                    "scores_ms": round(ms8_s, 4),
                    "scores_and_o_full_ms": round(ms8_f, 4),
                    "o_full_pass_ms": round(ms8_f - ms8_s, 4),
                    "achieved_TFLOPs": round(alg / (ms8 * 1e-3) / 1e12, 1),
                    "mfma_bf16_frac": round(alg / (ms8 * 1e-3) / 2.5e15, 4),
                    "note": "K and V as E4M3 bytes with one fp32 scale each, widened to bf16 "
                            "(exact) on the way into LDS; same FLOP count as the bf16 prefill"}
    del buf, inp, o_full
    # KV Bridging of 1,048,576 x 2048 hidden states, then decode over the cache.
    w = WORKLOADS["bridge_decode_bf16_1m"]
    g = torch.Generator(device="cuda").manual_seed(w.seed)
    m_rows, dm = w.ctx_len, w.d_model
    h = (torch.randn((m_rows, dm), generator=g, device="cuda") / dm ** 0.5).to(torch.bfloat16)
    wk = torch.randn((dm, w.head_dim), generator=g, device="cuda").to(torch.bfloat16)
    wv = torch.randn((dm, w.head_dim), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.empty((1, m_rows, w.head_dim), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    from kv_cache_reuse_hs2_amd.torch_api import pack_bridge_weights
    wp = pack_bridge_weights(wk, wv, dm)  # once per set of weights, outside the timing
    ms_pack = time_events(lambda: hs2.hs2_bridge_pack_weights(wk, wv, dm, wp), 5, 2)
    ms_u = time_events(lambda: hs2.hs2_bridge_kv(h, dm, wk, wv, k, v, w.head_dim, m_rows, dm),
                       max(3, steps // 5), 2)
    ms_b = time_events(lambda: hs2.hs2_bridge_kv_packed(h, dm, wp, k, v, w.head_dim, m_rows, dm),
                       max(3, steps // 5), 2)
    flop = 2.0 * m_rows * dm * 2 * w.head_dim
    byts = m_rows * dm * 2 + 2 * dm * w.head_dim * 2 + 2 * m_rows * w.head_dim * 2
    out["bridge_kv_1m_x_2048"] = {
        "ms": round(ms_b, 4), "achieved_TFLOPs": round(flop / (ms_b * 1e-3) / 1e12, 1),
        "mfma_bf16_frac": round(flop / (ms_b * 1e-3) / 2.5e15, 4),
        "hbm_GBps": round(byts / (ms_b * 1e-3) / 1e9, 1),
        "hbm_frac": round(byts / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "entry": "hs2_bridge_kv_packed (weights packed once)",
        "pack_weights_ms": round(ms_pack, 4),
        "hs2_bridge_kv_ms": round(ms_u, 4)}
    # Decode-time bridging: one new token for each of 4 sequences, written at
    # the end of their caches (the 1M-row K/V above serve as 4 caches of 256k).
    n_seq, cap_d = 4, m_rows // 4
    pos_d = torch.full((n_seq,), cap_d - 1, dtype=torch.int32, device="cuda")
    ms_d = time_events(lambda: hs2.hs2_bridge_kv_decode(h, dm, wp, n_seq, dm, pos_d, k, v,
                                                        cap_d * w.head_dim, cap_d),
                       steps, warmup)
    byts_d = 2 * dm * w.head_dim * 2 + n_seq * dm * 2 + 2 * n_seq * w.head_dim * 2
    out["bridge_kv_decode_b4_x_2048"] = {
        "us": round(ms_d * 1e3, 2), "hbm_GBps": round(byts_d / (ms_d * 1e-3) / 1e9, 1),
        "entry": "hs2_bridge_kv_decode", "algorithmic_bytes": byts_d}
    del h
    q = torch.randn((1, 1, w.n_heads, w.head_dim), generator=g, device="cuda").to(torch.bfloat16)
    desc = hs2.make_desc(batch=1, n_heads=w.n_heads, k_top=w.k_top, window=w.window)
    ctx = torch.tensor([m_rows], dtype=torch.int32, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    scores = torch.empty((1, 1, m_rows), **f32)
    ti = torch.empty((1, 1, w.k_top), dtype=torch.int32, device="cuda")
    tc = torch.empty((1, 1), dtype=torch.int32, device="cuda")
    o = torch.empty((1, 1, w.n_heads, w.head_dim), **f32)
    ws = torch.empty(hs2.hs2_workspace_size(desc, m_rows), dtype=torch.uint8, device="cuda")
    step = lambda: hs2.hs2_decode_step(desc, q, None, k, v, m_rows * w.head_dim, ctx, m_rows,  # noqa: E731
                                       scores, None, ti, tc, o, None, ws)
    ms = time_events(step, steps, warmup)
    ab = algorithmic_bytes(w)
    out["decode_bf16_1m_after_bridge"] = {
        "ms_per_step": round(ms, 5), "tokens_per_s": round(1 / (ms * 1e-3), 1),
        "step_hbm_GBps": round(ab["step"] / (ms * 1e-3) / 1e9, 1)}
    return out


def measured_traffic(kernels) -> float | None:
    """HBM bytes per launch of `kernels` from the committed counter summary
    (profiles/<workload>_traffic.json), or None when the sources the scoring
    kernel is built from (TRAFFIC_SOURCES) have changed since those counters
    were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"{WORKLOAD}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    csrc = os.path.join(ROOT, "kv_cache_reuse_hs2_amd", "csrc")
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        h.update(open(os.path.join(csrc, name), "rb").read())
    if h.hexdigest() != rec.get("source_sha256"):
        return None
    per = rec["bytes_per_dispatch"]
    if not all(k in per for k in kernels):
        return None
    return float(sum(per[k] for k in kernels))


def oracle_check(w, inp, buf, seq: int = 0) -> dict:
    """One sequence of the last timed step against the oracle (after the timed
    region): element-wise relative error of the scores, the selection's
    difference from the oracle's (only near-ties of the k-th score may
    differ), and the sparse output's error on the GPU's own selection."""
    import numpy as np

    import oracle

    sl = slice(seq, seq + 1)
    ctx = inp["ctx_len"][sl]
    n = int(ctx[0])
    s_or, _, _ = oracle.full_attn_scores(inp["q"][sl], inp["k"][sl], ctx, tile_q=1,
                                         sm_scale=w.sm_scale)
    s_gpu = buf.scores[sl].cpu().numpy()
    rel = np.abs(s_gpu[0, 0, :n].astype(np.float64) - s_or[0, 0, :n]) / np.maximum(
        np.abs(s_or[0, 0, :n]), 1e-30)
    top_or, cnt_or = oracle.select_topk_window(s_or, ctx, n_q=1, tile_q=1, k_top=w.k_top,
                                               window=w.window)
    top = buf.top_idx[sl].cpu().numpy()
    cnt = buf.top_cnt[sl].cpu().numpy()
    c = int(cnt_or[0, 0])
    diff = np.setxor1d(top[0, 0, :c], top_or[0, 0, :c])
    pe = oracle.pool_end(n - 1, w.window)
    pool = s_or[0, 0, :pe].astype(np.float64)
    tau = np.sort(pool)[::-1][c - 1] if c else 0.0
    near = bool(np.all(np.abs(pool[diff] - tau) <= 1e-4 * tau)) if diff.size else True
    o_or, _ = oracle.sparse_attention(inp["q"][sl], inp["k"][sl], inp["v"][sl], ctx, top, cnt,
                                      tile_q=1, window=w.window, sm_scale=w.sm_scale)
    o_err = float(np.abs(buf.o[sl].cpu().numpy() - o_or).max())
    return {"sequence": seq, "scores_max_rel_err": float(rel.max()),
            "top_cnt_equal": bool(cnt[0, 0] == c), "near_tie_swaps": int(diff.size // 2),
            "swaps_all_near_ties": near, "o_max_abs_err": o_err}


def cpu_baseline(w, inp, budget_s: float = 12.0) -> dict:
    """The oracle as it stands, on whole sequences of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle

    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    done, t0 = 0, time.perf_counter()
    while True:
        b = done % w.batch
        sl = slice(b, b + 1)
        ctx = inp["ctx_len"][sl]
        s, _, _ = oracle.full_attn_scores(inp["q"][sl], inp["k"][sl], ctx, tile_q=1,
                                          sm_scale=w.sm_scale)
        top, cnt = oracle.select_topk_window(s, ctx, n_q=1, tile_q=1, k_top=w.k_top,
                                             window=w.window)
        oracle.sparse_attention(inp["q"][sl], inp["k"][sl], inp["v"][sl], ctx, top, cnt,
                                tile_q=1, window=w.window, sm_scale=w.sm_scale)
        done += 1
        if time.perf_counter() - t0 >= budget_s or done >= 256:
            break
    dt = time.perf_counter() - t0
    del np
    return {"value": done / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} whole sequences ({w.ctx_len} keys, {w.n_heads} heads) of the same "
                      f"workload, one decode step each, fp64 NumPy, {dt:.1f} s"}


def cpu_baselines_all(budget_s: float = 8.0) -> dict:
    """The oracle timed on a bounded sample of every measured shape (host
    only, nothing on the GPU): whole decode sequences, prefill tiles with the
    context that ends at each tile, KV Bridging rows, and the sliding-window
    attention's queries.  Reported beside the GPU figures, never as targets."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from workloads import (WORKLOADS, bf16_bits_to_f32, make_bridge_inputs, make_decode_inputs,
                           make_prefill_inputs)

    threads = int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    out = {"cores": threads}

    def run(fn, n_max):
        done, t0 = 0, time.perf_counter()
        while done < n_max:
            fn(done)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        return done, time.perf_counter() - t0

    for name in ("decode_f32_4k", "decode_bf16_64k_b16", "decode_fp8_256k_b4"):
        w = WORKLOADS[name]
        inp = make_decode_inputs(w)
        if w.dtype == "fp8":
            inp["k"] = oracle.dequant_kv(inp["k_raw"], inp["k_scale"])
            inp["v"] = oracle.dequant_kv(inp["v_raw"], inp["v_scale"])

        def one(i, w=w, inp=inp):
            sl = slice(i % w.batch, i % w.batch + 1)
            ctx = inp["ctx_len"][sl]
            sc, _, _ = oracle.full_attn_scores(inp["q"][sl], inp["k"][sl], ctx, tile_q=1,
                                               sm_scale=w.sm_scale)
            top, cnt = oracle.select_topk_window(sc, ctx, n_q=1, tile_q=1, k_top=w.k_top,
                                                 window=w.window)
            oracle.sparse_attention(inp["q"][sl], inp["k"][sl], inp["v"][sl], ctx, top, cnt,
                                    tile_q=1, window=w.window, sm_scale=w.sm_scale)

        n, dt = run(one, 256)
        out[name] = {"value": round(n / dt, 3), "unit": "tokens/s",
                     "sample": f"{n} whole sequences, one decode step each, {dt:.1f} s"}
        del inp
    # Prefill: tiles of 64 queries, each with the context ending at its last query.
    w = WORKLOADS["prefill_bf16_128k_8k"]
    inp = make_prefill_inputs(w)
    rng = np.random.default_rng(7)
    tiles = rng.permutation(w.n_q // w.tile_q)

    def tile(i):
        t = int(tiles[i])
        q0, nk = t * w.tile_q, w.ctx_len - w.n_q + (t + 1) * w.tile_q
        ctx = np.array([nk], dtype=np.int32)
        qs = inp["q"][:, q0:q0 + w.tile_q]
        sc, _, _ = oracle.full_attn_scores(qs, inp["k"][:, :nk], ctx, tile_q=w.tile_q,
                                           sm_scale=w.sm_scale)
        top, cnt = oracle.select_topk_window(sc, ctx, n_q=w.tile_q, tile_q=w.tile_q,
                                             k_top=w.k_top, window=w.window)
        oracle.sparse_attention(qs, inp["k"][:, :nk], inp["v"][:, :nk], ctx, top, cnt,
                                tile_q=w.tile_q, window=w.window, sm_scale=w.sm_scale)

    n, dt = run(tile, len(tiles))
    out[w.name] = {"value": round(n * w.tile_q / dt, 2), "unit": "queries/s",
                   "sample": f"{n} seeded tiles of {w.tile_q} queries (scoring, selection and "
                             f"sparse layer), {dt:.1f} s"}
    # Sliding-window attention over the same queries, in blocks of 256.
    def swa(i):
        q0 = (i * 256) % w.n_q
        oracle.swa_attention(inp["q"][:, q0:q0 + 256], inp["k"], inp["v"],
                             np.array([w.ctx_len - w.n_q + q0 + 256], dtype=np.int32),
                             window=128, sm_scale=w.sm_scale)

    n, dt = run(swa, w.n_q // 256)
    out["swa_bf16_prefill_8k_w128"] = {"value": round(n * 256 / dt, 1), "unit": "queries/s",
                                       "sample": f"{n} blocks of 256 queries, window 128, "
                                                 f"{dt:.1f} s"}
    del inp
    # KV Bridging: 16,384-row blocks of the 1M x 2048 hidden states.
    wb = WORKLOADS["bridge_decode_bf16_1m"]
    bi = make_bridge_inputs(wb, rows=16384)
    h = bf16_bits_to_f32(bi["h_raw"])

    def bridge(i):
        oracle.bridge_kv(h, bi["w_k"], bi["w_v"])

    n, dt = run(bridge, 64)
    out["bridge_kv_1m_x_2048"] = {"value": round(n * 16384 / dt, 1), "unit": "rows/s",
                                  "sample": f"{n} blocks of 16,384 rows, {dt:.1f} s"}
    del np
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--graph", type=int, default=1, help="replay the step as a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extras", type=int, default=1,
                    help="also time batched decode, chunked prefill and KV Bridging")
    ap.add_argument("--cpu-baselines", action="store_true",
                    help="time the oracle on a sample of every shape (host only) and exit")
    ap.add_argument("--calibrate", action="store_true",
                    help="after timing, run a plain 256 MiB device copy (torch copy_) so that "
                         "HBM byte counters can be scaled by a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(decode shards by sequence with no exchange; see the design notes).",
              file=sys.stderr)
        return 2
    if args.cpu_baselines:
        print(json.dumps({"cpu_baselines": cpu_baselines_all()}), flush=True)
        return 0

    import numpy as np
    import torch

    import kv_cache_reuse_hs2_amd as hs2
    from kv_cache_reuse_hs2_amd.torch_api import (make_buffers, run_fused_step, run_scores,
                                                  run_select, run_sparse, run_step)
    from workloads import WORKLOADS, make_decode_inputs

    hs2.load()
    torch.cuda.set_device(0)
    w = WORKLOADS[WORKLOAD]
    t_gen = time.perf_counter()
    inp = make_decode_inputs(w)
    buf = make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                       sm_scale=w.sm_scale, dtype=w.dtype)
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    # Four distinct K/V caches (four full layers' caches, 2 GiB), used in turn,
    # so that no step finds its K left in the 256 MB memory-side cache by the
    # step before: in a model each full layer has a cache of its own.
    rot = [buf] + [make_buffers(inp, n_heads=w.n_heads, k_top=w.k_top, window=w.window,
                                sm_scale=w.sm_scale, dtype=w.dtype) for _ in range(3)]

    # Per-call timing (eager): HIP events on the stream the kernels run on.
    calls = {"scores": run_scores, "select": run_select, "sparse": run_sparse}
    for i in range(args.warmup):
        run_step(rot[i % 4])
    torch.cuda.synchronize()
    per_call = {k: [] for k in calls}
    for i in range(args.steps):
        bb = rot[i % 4]
        for name, fn in calls.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(bb)
            e1.record(stream)
            per_call[name].append((e0, e1))
    torch.cuda.synchronize()
    call_ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in per_call.items()}

    def capture(fn, bufs):
        """One HIP graph holding fn(b) for each b in bufs, in order."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for bb in bufs:
                fn(bb)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for bb in bufs:
                fn(bb)
        torch.cuda.synchronize()
        return g

    def timed(fn, bufs, n_steps, n_warm):
        """Milliseconds per step over exactly n_steps steps (after n_warm untimed
        ones), the steps cycling through bufs: from HIP graphs of GRAPH_ROUNDS
        rounds (a serving loop captures a whole model step, so the per-replay
        launch cost is not the layer's) plus one-step graphs for the rest, or
        eager calls when --graph 0.  Also returns the wall time of the region."""
        per = GRAPH_ROUNDS * len(bufs)
        if args.graph:
            g_many = capture(fn, bufs * GRAPH_ROUNDS)
            g_one = [capture(fn, [bb]) for bb in bufs]
            plan = lambda n: [g_many] * (n // per) + [g_one[i % len(bufs)] for i in range(n % per)]  # noqa: E731
            run = lambda gs: [g.replay() for g in gs]  # noqa: E731
        else:
            plan = lambda n: [bufs[i % len(bufs)] for i in range(n)]  # noqa: E731
            run = lambda bs: [fn(bb) for bb in bs]  # noqa: E731
        run(plan(n_warm))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_wall = time.perf_counter()
        e0.record(stream)
        run(plan(n_steps))
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n_steps, (time.perf_counter() - t_wall) * 1e3

    # The headline: the single-call step (hs2_decode_step) over the four caches.
    ms, wall_ms = timed(run_fused_step, rot, args.steps, args.warmup)
    # Beside it: the same step on one cache only (part of K then comes from the
    # memory-side cache), and the step issued as three calls over the four caches.
    ms_same, _ = timed(run_fused_step, [buf], args.steps, args.warmup)
    ms_3call, _ = timed(run_step, rot, args.steps, args.warmup)

    # Spread of single steps (after the timed region, not part of `value`):
    # each step replayed alone between two events, the caches in turn.
    def per_step(fn, n):
        gs = [capture(fn, [bb]) for bb in rot] if args.graph else None
        run1 = [g.replay for g in gs] if gs else [lambda bb=bb: fn(bb) for bb in rot]
        for i in range(4):
            run1[i]()
        ev = []
        for i in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run1[i % 4]()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
        return {"p10": round(float(np.percentile(us, 10)), 2),
                "median": round(float(np.median(us)), 2),
                "p90": round(float(np.percentile(us, 90)), 2), "n": n}

    step_spread = per_step(run_fused_step, max(args.steps, 20))
    check = oracle_check(w, inp, buf)
    del rot[1:]
    # Measured copy bandwidth of the box (a plain 1 GiB device copy, read +
    # write bytes), the practical ceiling the step's HBM rate is also set against.
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms_copy = time_events(lambda: dst.copy_(src), 10, 3)
    copy_gbs = 2 * (1 << 30) / (ms_copy * 1e-3) / 1e9
    del src, dst

    ab = algorithmic_bytes(w)
    tokens_s = w.batch / (ms * 1e-3)
    step_gbs = ab["step"] / (ms * 1e-3) / 1e9
    score_gbs = ab["scoring_call"] / (call_ms["scores"] * 1e-3) / 1e9
    out = {
        "metric": "sparse-attn decode tokens/s + HBM GB/s (% of peak) at 256k ctx, 1 GPU",
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD,
            "batch": w.batch,
            "ctx_len": w.ctx_len,
            "n_heads": w.n_heads,
            "kv_heads": 1,
            "head_dim": w.head_dim,
            "k_top": w.k_top,
            "window": w.window,
            "step": "hs2_decode_step (scoring + selection + sparse layer, one call), "
                    "over four distinct K/V caches in turn",
            "graph": bool(args.graph),
            "graph_steps": GRAPH_ROUNDS * 4 if args.graph else 0,
            "step_algorithmic_MiB": round(ab["step"] / MIB, 2),
            "step_hbm_GBps": round(step_gbs, 1),
            "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
            "call_ms": {k: round(v, 5) for k, v in call_ms.items()},
            "ms_per_step_same_cache": round(ms_same, 5),
            "tokens_per_s_same_cache": round(w.batch / (ms_same * 1e-3), 1),
            "ms_per_step_three_calls": round(ms_3call, 5),
            "wall_ms_timed_region": round(wall_ms, 3),
            "single_step_us": step_spread,
            "hbm_copy_GBps": round(copy_gbs, 1),
            "step_hbm_frac_of_copy": round(step_gbs / copy_gbs, 4),
            "scoring_call_hbm_frac_of_copy": round(score_gbs / copy_gbs, 4),
            "oracle_check": check,
        },
        "roofline": {
            "kernel": f"{SCORE_KERNEL} (hs2_full_attn_scores: K read once)",
            "bound": "hbm",
            "achieved": round(score_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(score_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic([SCORE_KERNEL]),
            "algorithmic_bytes_per_launch": ab["scoring_call"],
        },
    }
    if args.extras:
        del buf
        out["extras"] = extra_measurements(args.steps, args.warmup)
        out["extras"]["decode_bf16_256k_b4_shared_selection"] = sparse_layer_measurements(
            args.steps, args.warmup)
        out["extras"]["decode_fp8_256k_b4"] = fp8_measurements(args.steps, args.warmup)
        out["extras"]["decode_bf16_256k_b4_block_vs_token"] = block_measurements(args.steps,
                                                                                 args.warmup)
        out["extras"]["swa_bf16_prefill_8k_w128"] = swa_measurements(args.steps, args.warmup)
        out["extras"]["decode_bf16_256k_b4_full_layer"] = full_output_measurements(args.steps,
                                                                                  args.warmup)
        out["extras"]["mfma_calibration"] = mfma_calibration(args.steps, args.warmup)
    if args.calibrate:
        src = torch.empty(256 * MIB, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["config"]["calibration_copy_bytes"] = 256 * MIB
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
