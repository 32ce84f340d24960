"""Python binding of libhs2: HySparse2 inner-level KV Reuse kernels for MI355X.

Thin ctypes layer over the C ABI declared in ``include/hs2.h``: it only turns
torch tensors into device pointers and the current HIP stream, and turns
status codes into exceptions.  Every step of the computation runs in the HIP
kernels of ``libhs2.so``; there is no fallback.  If the library is missing,
loading raises.

PyTorch is used for device memory and streams only.  It is imported before
the library is loaded, so that libhs2 binds to the same HIP runtime as torch
(both carry the soname ``libamdhip64.so.7``).
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhs2.so")

HS2_F32 = 0
HS2_BF16 = 1
HS2_FP8_E4M3 = 2
HS2_OK, HS2_EINVAL, HS2_EUNSUPPORTED, HS2_EALIGN, HS2_EWORKSPACE, HS2_EHIP = range(6)

EXPORTS = (
    "hs2_workspace_size",
    "hs2_full_attn_scores",
    "hs2_select_topk_window",
    "hs2_select_topk_blocks",
    "hs2_sparse_attn_gather",
    "hs2_sparse_layers_workspace_size",
    "hs2_sparse_attn_gather_layers",
    "hs2_decode_step",
    "hs2_decode_step_blocks",
    "hs2_decode_step_noalloc",
    "hs2_swa_attention",
    "hs2_bridge_kv",
    "hs2_bridge_packed_bytes",
    "hs2_bridge_pack_weights",
    "hs2_bridge_kv_packed",
    "hs2_bridge_kv_decode",
    "hs2_status_string",
)


class hs2_attn_desc(ctypes.Structure):
    """Mirror of ``hs2_attn_desc`` in include/hs2.h."""

    _fields_ = [
        ("batch", ctypes.c_int),
        ("n_q", ctypes.c_int),
        ("n_heads", ctypes.c_int),
        ("head_dim", ctypes.c_int),
        ("tile_q", ctypes.c_int),
        ("k_top", ctypes.c_int),
        ("window", ctypes.c_int),
        ("causal", ctypes.c_int),
        ("sm_scale", ctypes.c_float),
        ("dtype", ctypes.c_int),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


class HS2Error(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {hs2_status_string(status)}")


_lib = None
_vp, _i64, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
_desc_p = ctypes.POINTER(hs2_attn_desc)


def load(path: str | None = None):
    """Load libhs2.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- binds the HIP runtime torch ships

    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"libhs2.so not built ({p}); run python -m kv_cache_reuse_hs2_amd.build_lib")
    lib = ctypes.CDLL(p)
    lib.hs2_workspace_size.argtypes = [_desc_p, _int]
    lib.hs2_workspace_size.restype = _sz
    lib.hs2_full_attn_scores.argtypes = [_desc_p, _vp, _vp, _vp, _i64, _vp, _int, _vp, _vp, _vp,
                                         _vp, _sz, _vp]
    lib.hs2_full_attn_scores.restype = _int
    lib.hs2_select_topk_window.argtypes = [_desc_p, _vp, _vp, _int, _vp, _vp, _vp, _sz, _vp]
    lib.hs2_select_topk_window.restype = _int
    lib.hs2_select_topk_blocks.argtypes = [_desc_p, _int, _vp, _vp, _int, _vp, _vp, _vp, _sz, _vp]
    lib.hs2_select_topk_blocks.restype = _int
    lib.hs2_sparse_attn_gather.argtypes = [_desc_p, _vp, _vp, _vp, _i64, _vp, _int, _vp, _vp,
                                           _vp, _vp, _vp, _sz, _vp]
    lib.hs2_sparse_attn_gather.restype = _int
    lib.hs2_sparse_layers_workspace_size.argtypes = [_desc_p, _int]
    lib.hs2_sparse_layers_workspace_size.restype = _sz
    lib.hs2_sparse_attn_gather_layers.argtypes = [_desc_p, _int, _vp, _vp, _vp, _i64, _vp, _int,
                                                  _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    lib.hs2_sparse_attn_gather_layers.restype = _int
    lib.hs2_decode_step.argtypes = [_desc_p, _vp, _vp, _vp, _vp, _i64, _vp, _int, _vp, _vp, _vp,
                                    _vp, _vp, _vp, _vp, _sz, _vp]
    lib.hs2_decode_step.restype = _int
    lib.hs2_decode_step_blocks.argtypes = [_desc_p, _int, _vp, _vp, _vp, _vp, _i64, _vp, _int,
                                           _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    lib.hs2_decode_step_blocks.restype = _int
    lib.hs2_decode_step_noalloc.argtypes = [_desc_p, _vp, _vp, _vp, _vp, _i64, _vp, _int, _vp,
                                            _vp, _vp, _vp, _vp, _vp, _vp]
    lib.hs2_decode_step_noalloc.restype = _int
    lib.hs2_swa_attention.argtypes = [_desc_p, _vp, _vp, _vp, _i64, _vp, _int, _vp, _int, _vp,
                                      _vp]
    lib.hs2_swa_attention.restype = _int
    lib.hs2_bridge_packed_bytes.argtypes = [_int, _int]
    lib.hs2_bridge_packed_bytes.restype = _sz
    lib.hs2_bridge_pack_weights.argtypes = [_vp, _vp, _int, _int, _vp, _vp]
    lib.hs2_bridge_pack_weights.restype = _int
    lib.hs2_bridge_kv.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp, _i64, _int, _int, _int, _vp]
    lib.hs2_bridge_kv_packed.argtypes = [_vp, _i64, _vp, _vp, _vp, _i64, _int, _int, _int, _vp]
    lib.hs2_bridge_kv_packed.restype = _int
    lib.hs2_bridge_kv_decode.argtypes = [_vp, _i64, _vp, _int, _int, _int, _vp, _vp, _vp, _i64,
                                         _int, _vp]
    lib.hs2_bridge_kv_decode.restype = _int
    lib.hs2_bridge_kv.restype = _int
    lib.hs2_status_string.argtypes = [_int]
    lib.hs2_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def make_desc(*, batch, n_heads, n_q=1, tile_q=1, k_top=1024, window=128, sm_scale=None,
              dtype=HS2_BF16, head_dim=128, causal=1, k_scale=1.0,
              v_scale=1.0) -> hs2_attn_desc:
    if sm_scale is None:
        sm_scale = head_dim ** -0.5
    return hs2_attn_desc(batch, n_q, n_heads, head_dim, tile_q, k_top, window, causal,
                         float(sm_scale), int(dtype), float(k_scale), float(v_scale))


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _nbytes(ws) -> int:
    if ws is None:
        return 0
    return ws.numel() * ws.element_size()


def _check(status: int, call: str) -> None:
    if status != HS2_OK:
        raise HS2Error(status, call)


def hs2_status_string(status: int) -> str:
    return load().hs2_status_string(int(status)).decode()


def hs2_workspace_size(desc: hs2_attn_desc, kv_capacity: int) -> int:
    return int(load().hs2_workspace_size(ctypes.byref(desc), int(kv_capacity)))


def hs2_full_attn_scores(desc, q, k, v, kv_stride, ctx_len, kv_capacity, scores, o_full=None,
                         lse=None, ws=None, stream=None) -> None:
    st = load().hs2_full_attn_scores(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), int(kv_stride),
                                     _ptr(ctx_len), int(kv_capacity), _ptr(scores), _ptr(o_full),
                                     _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream))
    _check(st, "hs2_full_attn_scores")


def hs2_select_topk_window(desc, scores, ctx_len, kv_capacity, top_idx, top_cnt, ws=None,
                           stream=None) -> None:
    st = load().hs2_select_topk_window(ctypes.byref(desc), _ptr(scores), _ptr(ctx_len),
                                       int(kv_capacity), _ptr(top_idx), _ptr(top_cnt), _ptr(ws),
                                       _nbytes(ws), _stream(stream))
    _check(st, "hs2_select_topk_window")


def hs2_select_topk_blocks(desc, block_size, scores, ctx_len, kv_capacity, top_idx, top_cnt,
                           ws=None, stream=None) -> None:
    st = load().hs2_select_topk_blocks(ctypes.byref(desc), int(block_size), _ptr(scores),
                                       _ptr(ctx_len), int(kv_capacity), _ptr(top_idx),
                                       _ptr(top_cnt), _ptr(ws), _nbytes(ws), _stream(stream))
    _check(st, "hs2_select_topk_blocks")


def hs2_sparse_attn_gather(desc, q, k, v, kv_stride, ctx_len, kv_capacity, top_idx, top_cnt, o,
                           lse=None, ws=None, stream=None) -> None:
    st = load().hs2_sparse_attn_gather(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                       int(kv_stride), _ptr(ctx_len), int(kv_capacity),
                                       _ptr(top_idx), _ptr(top_cnt), _ptr(o), _ptr(lse), _ptr(ws),
                                       _nbytes(ws), _stream(stream))
    _check(st, "hs2_sparse_attn_gather")


def hs2_sparse_layers_workspace_size(desc, n_layers) -> int:
    return int(load().hs2_sparse_layers_workspace_size(ctypes.byref(desc), int(n_layers)))


def hs2_sparse_attn_gather_layers(desc, n_layers, q_layers, k, v, kv_stride, ctx_len,
                                  kv_capacity, top_idx, top_cnt, o_layers, lse_layers=None,
                                  ws=None, stream=None) -> None:
    st = load().hs2_sparse_attn_gather_layers(
        ctypes.byref(desc), int(n_layers), _ptr(q_layers), _ptr(k), _ptr(v), int(kv_stride),
        _ptr(ctx_len), int(kv_capacity), _ptr(top_idx), _ptr(top_cnt), _ptr(o_layers),
        _ptr(lse_layers), _ptr(ws), _nbytes(ws), _stream(stream))
    _check(st, "hs2_sparse_attn_gather_layers")


def hs2_decode_step(desc, q, q_sparse, k, v, kv_stride, ctx_len, kv_capacity, scores, lse_full,
                    top_idx, top_cnt, o, lse=None, ws=None, stream=None) -> None:
    st = load().hs2_decode_step(ctypes.byref(desc), _ptr(q), _ptr(q_sparse), _ptr(k), _ptr(v),
                                int(kv_stride), _ptr(ctx_len), int(kv_capacity), _ptr(scores),
                                _ptr(lse_full), _ptr(top_idx), _ptr(top_cnt), _ptr(o), _ptr(lse),
                                _ptr(ws), _nbytes(ws), _stream(stream))
    _check(st, "hs2_decode_step")


def hs2_decode_step_blocks(desc, block_size, q, q_sparse, k, v, kv_stride, ctx_len, kv_capacity,
                           scores, lse_full, top_idx, top_cnt, o, lse=None, ws=None,
                           stream=None) -> None:
    st = load().hs2_decode_step_blocks(ctypes.byref(desc), int(block_size), _ptr(q),
                                       _ptr(q_sparse), _ptr(k), _ptr(v), int(kv_stride),
                                       _ptr(ctx_len), int(kv_capacity), _ptr(scores),
                                       _ptr(lse_full), _ptr(top_idx), _ptr(top_cnt), _ptr(o),
                                       _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream))
    _check(st, "hs2_decode_step_blocks")


def hs2_decode_step_noalloc(desc, q, q_sparse, k, v, kv_stride, ctx_len, kv_capacity, scores,
                            lse_full, top_idx, top_cnt, o, lse=None, stream=None) -> None:
    st = load().hs2_decode_step_noalloc(ctypes.byref(desc), _ptr(q), _ptr(q_sparse), _ptr(k),
                                        _ptr(v), int(kv_stride), _ptr(ctx_len), int(kv_capacity),
                                        _ptr(scores), _ptr(lse_full), _ptr(top_idx),
                                        _ptr(top_cnt), _ptr(o), _ptr(lse), _stream(stream))
    _check(st, "hs2_decode_step_noalloc")


def hs2_swa_attention(desc, q, k, v, kv_stride, ctx_len, kv_capacity, o, o_dtype=HS2_F32,
                      lse=None, stream=None) -> None:
    st = load().hs2_swa_attention(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), int(kv_stride),
                                  _ptr(ctx_len), int(kv_capacity), _ptr(o), int(o_dtype),
                                  _ptr(lse), _stream(stream))
    _check(st, "hs2_swa_attention")


def hs2_bridge_packed_bytes(d_model, head_dim=128) -> int:
    return int(load().hs2_bridge_packed_bytes(int(d_model), int(head_dim)))


def hs2_bridge_pack_weights(w_k, w_v, d_model, w_packed, head_dim=128, stream=None) -> None:
    st = load().hs2_bridge_pack_weights(_ptr(w_k), _ptr(w_v), int(d_model), int(head_dim),
                                        _ptr(w_packed), _stream(stream))
    _check(st, "hs2_bridge_pack_weights")


def hs2_bridge_kv(h, ldh, w_k, w_v, k_out, v_out, ld_kv, M, d_model, head_dim=128,
                  stream=None) -> None:
    st = load().hs2_bridge_kv(_ptr(h), int(ldh), _ptr(w_k), _ptr(w_v), _ptr(k_out), _ptr(v_out),
                              int(ld_kv), int(M), int(d_model), int(head_dim), _stream(stream))
    _check(st, "hs2_bridge_kv")


def hs2_bridge_kv_packed(h, ldh, w_packed, k_out, v_out, ld_kv, M, d_model, head_dim=128,
                         stream=None) -> None:
    st = load().hs2_bridge_kv_packed(_ptr(h), int(ldh), _ptr(w_packed), _ptr(k_out), _ptr(v_out),
                                     int(ld_kv), int(M), int(d_model), int(head_dim),
                                     _stream(stream))
    _check(st, "hs2_bridge_kv_packed")


def hs2_bridge_kv_decode(h, ldh, w_packed, rows, d_model, pos, k_cache, v_cache, kv_stride,
                         kv_capacity, head_dim=128, stream=None) -> None:
    st = load().hs2_bridge_kv_decode(_ptr(h), int(ldh), _ptr(w_packed), int(rows), int(d_model),
                                     int(head_dim), _ptr(pos), _ptr(k_cache), _ptr(v_cache),
                                     int(kv_stride), int(kv_capacity), _stream(stream))
    _check(st, "hs2_bridge_kv_decode")
