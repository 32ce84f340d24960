"""Torch-side plumbing around the C ABI: device buffers and a decode step.

Nothing here computes: it allocates outputs and workspace with torch and
calls the libhs2 entry points in order on the current stream.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import (HS2_BF16, HS2_F32, HS2_FP8_E4M3, hs2_attn_desc, hs2_bridge_pack_weights,
               hs2_bridge_packed_bytes, hs2_decode_step, hs2_decode_step_blocks,
               hs2_full_attn_scores, hs2_select_topk_blocks, hs2_select_topk_window,
               hs2_sparse_attn_gather, hs2_sparse_attn_gather_layers,
               hs2_sparse_layers_workspace_size, hs2_workspace_size, make_desc)


def to_device(arr: np.ndarray, device="cuda") -> torch.Tensor:
    """Copy a host array to the device, keeping raw bfloat16 bits as int16."""
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


@dataclasses.dataclass
class DecodeBuffers:
    """Device inputs and outputs of one decode step (or query-group step)."""

    desc: hs2_attn_desc
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    ctx_len: torch.Tensor
    cap: int
    scores: torch.Tensor
    top_idx: torch.Tensor
    top_cnt: torch.Tensor
    o: torch.Tensor
    lse_full: torch.Tensor
    lse: torch.Tensor
    ws: torch.Tensor

    @property
    def kv_stride(self) -> int:
        return self.k.shape[1] * self.k.shape[2]


def make_buffers(inp: dict, *, n_heads: int, k_top: int, window: int, sm_scale: float,
                 dtype: str, n_q: int = 1, tile_q: int = 1, device="cuda") -> DecodeBuffers:
    """Upload generator output (see ``workloads``) and allocate the outputs.

    dtype "f32", "bf16" or "fp8" (E4M3 K/V bytes with inp["k_scale"] and
    inp["v_scale"], bf16 queries)."""
    bsz = inp["ctx_len"].shape[0]
    cap = int(inp["capacity"])
    code = {"f32": HS2_F32, "bf16": HS2_BF16, "fp8": HS2_FP8_E4M3}[dtype]
    scales = {}
    if dtype == "fp8":
        scales = dict(k_scale=float(inp["k_scale"]), v_scale=float(inp["v_scale"]))
    desc = make_desc(batch=bsz, n_heads=n_heads, n_q=n_q, tile_q=tile_q, k_top=k_top,
                     window=window, sm_scale=sm_scale, dtype=code, **scales)
    tiles = n_q // tile_q
    nbytes = hs2_workspace_size(desc, cap)
    if nbytes == 0:
        raise ValueError("descriptor rejected by hs2_workspace_size")
    f32 = dict(dtype=torch.float32, device=device)
    i32 = dict(dtype=torch.int32, device=device)
    return DecodeBuffers(
        desc=desc,
        q=to_device(inp["q_raw"], device),
        k=to_device(inp["k_raw"], device),
        v=to_device(inp["v_raw"], device),
        ctx_len=to_device(inp["ctx_len"].astype(np.int32), device),
        cap=cap,
        scores=torch.zeros((bsz, tiles, cap), **f32),
        top_idx=torch.empty((bsz, tiles, max(k_top, 1)), **i32),
        top_cnt=torch.empty((bsz, tiles), **i32),
        o=torch.empty((bsz, n_q, n_heads, 128), **f32),
        lse_full=torch.empty((bsz, n_q, n_heads), **f32),
        lse=torch.empty((bsz, n_q, n_heads), **f32),
        ws=torch.empty(nbytes, dtype=torch.uint8, device=device),
    )


def run_scores(buf: DecodeBuffers, stream=None) -> None:
    hs2_full_attn_scores(buf.desc, buf.q, buf.k, None, buf.kv_stride, buf.ctx_len, buf.cap,
                         buf.scores, None, buf.lse_full, buf.ws, stream)


def run_scores_full(buf: DecodeBuffers, o_full: torch.Tensor, stream=None) -> None:
    """Scoring that also writes the full layer's own output o_full, fp32
    [B][n_q][H][128] (decode: n_q = 1, so [B][H][128] is the same memory)."""
    hs2_full_attn_scores(buf.desc, buf.q, buf.k, buf.v, buf.kv_stride, buf.ctx_len, buf.cap,
                         buf.scores, o_full, buf.lse_full, buf.ws, stream)


def run_select(buf: DecodeBuffers, scores: torch.Tensor | None = None, stream=None) -> None:
    hs2_select_topk_window(buf.desc, buf.scores if scores is None else scores, buf.ctx_len,
                           buf.cap, buf.top_idx, buf.top_cnt, buf.ws, stream)


def run_select_blocks(buf: DecodeBuffers, block: int, scores: torch.Tensor | None = None,
                      stream=None) -> None:
    hs2_select_topk_blocks(buf.desc, block, buf.scores if scores is None else scores,
                           buf.ctx_len, buf.cap, buf.top_idx, buf.top_cnt, buf.ws, stream)


def run_sparse(buf: DecodeBuffers, q: torch.Tensor | None = None, top_idx=None, top_cnt=None,
               stream=None) -> None:
    hs2_sparse_attn_gather(buf.desc, buf.q if q is None else q, buf.k, buf.v, buf.kv_stride,
                           buf.ctx_len, buf.cap, buf.top_idx if top_idx is None else top_idx,
                           buf.top_cnt if top_cnt is None else top_cnt, buf.o, buf.lse, buf.ws,
                           stream)


def run_step(buf: DecodeBuffers, stream=None) -> None:
    """One pass of the hot path as three calls: scoring, selection, sparse layer."""
    run_scores(buf, stream)
    run_select(buf, stream=stream)
    run_sparse(buf, stream=stream)


def run_fused_step(buf: DecodeBuffers, q_sparse: torch.Tensor | None = None, stream=None) -> None:
    """One pass of the hot path through the single-call entry point."""
    hs2_decode_step(buf.desc, buf.q, q_sparse, buf.k, buf.v, buf.kv_stride, buf.ctx_len, buf.cap,
                    buf.scores, buf.lse_full, buf.top_idx, buf.top_cnt, buf.o, buf.lse, buf.ws,
                    stream)


def run_fused_step_blocks(buf: DecodeBuffers, block: int, q_sparse: torch.Tensor | None = None,
                          stream=None) -> None:
    """One pass of the path with block-level selection, in a single call."""
    hs2_decode_step_blocks(buf.desc, block, buf.q, q_sparse, buf.k, buf.v, buf.kv_stride,
                           buf.ctx_len, buf.cap, buf.scores, buf.lse_full, buf.top_idx,
                           buf.top_cnt, buf.o, buf.lse, buf.ws, stream)


def pack_bridge_weights(w_k: torch.Tensor, w_v: torch.Tensor, d_model: int,
                        stream=None) -> torch.Tensor:
    """Device buffer holding [W_K | W_V] packed for hs2_bridge_kv."""
    n = hs2_bridge_packed_bytes(d_model)
    if n == 0:
        raise ValueError(f"unsupported d_model {d_model}")
    w_packed = torch.empty(n // 2, dtype=torch.int16, device=w_k.device)
    hs2_bridge_pack_weights(w_k, w_v, d_model, w_packed, stream=stream)
    return w_packed


def run_sparse_layers(buf: DecodeBuffers, q_layers: torch.Tensor, stream=None):
    """The sparse layers that share buf's selection: q_layers [L][B][1][H][D]
    (bf16 bits); returns (o_layers [L][B][1][H][D], lse_layers [L][B][1][H])."""
    n_layers = q_layers.shape[0]
    nbytes = hs2_sparse_layers_workspace_size(buf.desc, n_layers)
    if nbytes == 0:
        raise ValueError("descriptor rejected by hs2_sparse_layers_workspace_size")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=buf.k.device)
    o = torch.empty((n_layers,) + tuple(buf.o.shape), dtype=torch.float32, device=buf.k.device)
    lse = torch.empty((n_layers,) + tuple(buf.lse.shape), dtype=torch.float32, device=buf.k.device)
    hs2_sparse_attn_gather_layers(buf.desc, n_layers, q_layers, buf.k, buf.v, buf.kv_stride,
                                  buf.ctx_len, buf.cap, buf.top_idx, buf.top_cnt, o, lse, ws,
                                  stream)
    return o, lse
