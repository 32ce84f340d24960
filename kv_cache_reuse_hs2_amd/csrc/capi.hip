// C ABI entry points of libhs2: host-side validation (validate.cpp), then
// kernel dispatch.  Every argument check happens before the first enqueue, so
// a call that returns an error has enqueued nothing.
#include <string.h>

#include "hs2_internal.h"
#include "validate.h"

namespace hs2 {

hipError_t launch_bridge_pack(const uint16_t* w_k, const uint16_t* w_v, uint16_t* w_packed,
                              int d_model, hipStream_t st);
hipError_t launch_bridge_decode(const uint16_t* h, int64_t ldh, const uint16_t* w_packed,
                                int rows, int d_model, const int32_t* pos, uint16_t* k_cache,
                                uint16_t* v_cache, int64_t kv_stride, int cap, hipStream_t st);
hipError_t launch_bridge(const uint16_t* h, int64_t ldh, const uint16_t* w_packed,
                         const uint16_t* w_k, const uint16_t* w_v, uint16_t* k_out,
                         uint16_t* v_out, int64_t ld_kv, int M, int d_model, hipStream_t st);

namespace {

hs2_status launched(hipError_t e) { return e == hipSuccess ? HS2_OK : HS2_EHIP; }

}  // namespace
}  // namespace hs2

using namespace hs2;

extern "C" {

size_t hs2_workspace_size(const hs2_attn_desc* desc, int kv_capacity) {
  return workspace_bytes(desc, kv_capacity);
}

hs2_status hs2_full_attn_scores(const hs2_attn_desc* desc, const void* q, const void* k,
                                const void* v, int64_t kv_stride, const int32_t* ctx_len,
                                int kv_capacity, float* scores, float* o_full, float* lse,
                                void* ws, size_t ws_bytes, hs2_stream_t stream) {
  const hs2_status s = validate_full_attn_scores(desc, q, k, v, kv_stride, ctx_len, kv_capacity,
                                                 scores, o_full, lse, ws, ws_bytes);
  if (s != HS2_OK) return s;
  (void)hipGetLastError();
  const WsLayout l = ws_layout(*desc, kv_capacity);
  if (o_full != nullptr && is_prefill(*desc)) {
    // Scores (and the per-row statistics, kept in the workspace), then the
    // output pass that reads those statistics.
    const hipError_t e = launch_prefill_scores(*desc, q, k, kv_stride, ctx_len, kv_capacity,
                                               scores, lse, static_cast<char*>(ws) + l.score,
                                               false, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return launched(e);
    return launched(launch_prefill_out(*desc, q, k, v, kv_stride, ctx_len, kv_capacity, o_full,
                                       static_cast<char*>(ws) + l.score,
                                       static_cast<hipStream_t>(stream)));
  }
  if (o_full != nullptr)
    return launched(launch_score_full(*desc, q, k, v, kv_stride, ctx_len, kv_capacity, scores,
                                      o_full, lse, static_cast<char*>(ws) + l.score,
                                      static_cast<hipStream_t>(stream)));
  if (is_prefill(*desc))
    return launched(launch_prefill_scores(*desc, q, k, kv_stride, ctx_len, kv_capacity, scores,
                                          lse, static_cast<char*>(ws) + l.score, false,
                                          static_cast<hipStream_t>(stream)));
  return launched(launch_score_decode(
      *desc, q, k, kv_stride, ctx_len, kv_capacity, scores, lse, static_cast<char*>(ws) + l.score,
      reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + l.sync), false,
      static_cast<hipStream_t>(stream)));
}

hs2_status hs2_select_topk_window(const hs2_attn_desc* desc, const float* scores,
                                  const int32_t* ctx_len, int kv_capacity, int32_t* top_idx,
                                  int32_t* top_cnt, void* ws, size_t ws_bytes,
                                  hs2_stream_t stream) {
  const hs2_status s = validate_select_topk_window(desc, scores, ctx_len, kv_capacity, top_idx,
                                                   top_cnt, ws, ws_bytes);
  if (s != HS2_OK) return s;
  (void)hipGetLastError();
  const WsLayout l = ws_layout(*desc, kv_capacity);
  return launched(launch_select(*desc, scores, ctx_len, kv_capacity, top_idx, top_cnt,
                                static_cast<char*>(ws) + l.select, nullptr, true,
                                static_cast<hipStream_t>(stream)));
}

hs2_status hs2_select_topk_blocks(const hs2_attn_desc* desc, int block_size, const float* scores,
                                  const int32_t* ctx_len, int kv_capacity, int32_t* top_idx,
                                  int32_t* top_cnt, void* ws, size_t ws_bytes,
                                  hs2_stream_t stream) {
  const hs2_status s = validate_select_topk_blocks(desc, block_size, scores, ctx_len,
                                                   kv_capacity, top_idx, top_cnt, ws, ws_bytes);
  if (s != HS2_OK) return s;
  (void)hipGetLastError();
  const WsLayout l = ws_layout(*desc, kv_capacity);
  return launched(launch_select_blocks(*desc, block_size, scores, ctx_len, kv_capacity, top_idx,
                                       top_cnt, static_cast<char*>(ws) + l.select,
                                       static_cast<hipStream_t>(stream)));
}

hs2_status hs2_sparse_attn_gather(const hs2_attn_desc* desc, const void* q, const void* k,
                                  const void* v, int64_t kv_stride, const int32_t* ctx_len,
                                  int kv_capacity, const int32_t* top_idx,
                                  const int32_t* top_cnt, float* o, float* lse, void* ws,
                                  size_t ws_bytes, hs2_stream_t stream) {
  const hs2_status s = validate_sparse_attn_gather(desc, q, k, v, kv_stride, ctx_len, kv_capacity,
                                                   top_idx, top_cnt, o, lse, ws, ws_bytes);
  if (s != HS2_OK) return s;
  (void)hipGetLastError();
  const WsLayout l = ws_layout(*desc, kv_capacity);
  if (is_prefill(*desc))
    return launched(launch_prefill_sparse(*desc, q, k, v, kv_stride, ctx_len, kv_capacity, top_idx,
                                          top_cnt, o, lse, static_cast<hipStream_t>(stream)));
  return launched(launch_sparse(*desc, q, k, v, kv_stride, ctx_len, kv_capacity, top_idx, top_cnt,
                                o, lse, static_cast<char*>(ws) + l.sparse,
                                static_cast<hipStream_t>(stream)));
}

size_t hs2_sparse_layers_workspace_size(const hs2_attn_desc* desc, int n_layers) {
  return layers_workspace_bytes(desc, n_layers);
}

hs2_status hs2_sparse_attn_gather_layers(const hs2_attn_desc* desc, int n_layers,
                                         const void* q_layers, const void* k, const void* v,
                                         int64_t kv_stride, const int32_t* ctx_len,
                                         int kv_capacity, const int32_t* top_idx,
                                         const int32_t* top_cnt, float* o_layers,
                                         float* lse_layers, void* ws, size_t ws_bytes,
                                         hs2_stream_t stream) {
  const hs2_status s = validate_sparse_attn_gather_layers(
      desc, n_layers, q_layers, k, v, kv_stride, ctx_len, kv_capacity, top_idx, top_cnt, o_layers,
      lse_layers, ws, ws_bytes);
  if (s != HS2_OK) return s;
  (void)hipGetLastError();
  return launched(launch_sparse_layers(*desc, n_layers, q_layers, k, v, kv_stride, ctx_len,
                                       kv_capacity, top_idx, top_cnt, o_layers, lse_layers,
                                       static_cast<char*>(ws), static_cast<hipStream_t>(stream)));
}

hs2_status hs2_decode_step(const hs2_attn_desc* desc, const void* q, const void* q_sparse,
                           const void* k, const void* v, int64_t kv_stride,
                           const int32_t* ctx_len, int kv_capacity, float* scores,
                           float* lse_full, int32_t* top_idx, int32_t* top_cnt, float* o,
                           float* lse, void* ws, size_t ws_bytes, hs2_stream_t stream) {
  const hs2_status s = validate_step(desc, q, q_sparse, k, v, kv_stride, ctx_len, kv_capacity,
                                     scores, lse_full, top_idx, top_cnt, o, lse, ws, ws_bytes);
  if (s != HS2_OK) return s;
  if (q_sparse == nullptr) q_sparse = q;
  (void)hipGetLastError();
  const WsLayout l = ws_layout(*desc, kv_capacity);
  char* w = static_cast<char*>(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // The scoring pass also builds the selector's histogram (decode, and bf16
  // or E4M3 prefill), and the one-pass decode kernel also runs the
  // selector's candidate filter.
  const bool pf = is_prefill(*desc);
  const bool fuse = !pf || desc->dtype != HS2_F32;
  const SelectWs sw = select_ws(*desc, kv_capacity);
  FilterArgs filt{};
  filt.cnt = reinterpret_cast<uint32_t*>(w + l.select + sw.cnt_off);
  filt.meta = reinterpret_cast<uint32_t*>(w + l.select + sw.meta_off);
  filt.list = reinterpret_cast<uint2*>(w + l.select + sw.list_off);
  filt.nslices = select_slices(kv_capacity);
  filt.k_top = desc->k_top;
  bool filtered = false;
  hipError_t e =
      pf ? launch_prefill_scores(*desc, q, k, kv_stride, ctx_len, kv_capacity, scores, lse_full,
                                 w + l.score, fuse, st)
         : launch_score_decode(*desc, q, k, kv_stride, ctx_len, kv_capacity, scores, lse_full,
                               w + l.score, reinterpret_cast<uint64_t*>(w + l.sync), fuse, st,
                               fuse ? &filt : nullptr, &filtered);
  if (e != hipSuccess) return HS2_EHIP;
  const size_t hist_off = pf ? prefill_ws(*desc, kv_capacity).hist_off
                             : score_ws(*desc, kv_capacity).hist_off;
  uint32_t* hist = fuse ? reinterpret_cast<uint32_t*>(w + l.score + hist_off) : nullptr;
  // MFMA decode: the final selection runs inside the sparse layer's kernel
  // (with the fp32 segments' 256 threads it was slower than its own launch).
  const bool tail = !pf && desc->dtype != HS2_F32;
  if (!filtered) {
    e = launch_select(*desc, scores, ctx_len, kv_capacity, top_idx, top_cnt, w + l.select, hist,
                      !tail, st);
    if (e != hipSuccess) return HS2_EHIP;
  }
  if (pf)
    return launched(launch_prefill_sparse(*desc, q_sparse, k, v, kv_stride, ctx_len, kv_capacity,
                                          top_idx, top_cnt, o, lse, st));
  if (tail)
    return launched(launch_decode_tail(*desc, q_sparse, k, v, kv_stride, ctx_len, kv_capacity,
                                       hist, w + l.select, top_idx, top_cnt, o, lse, w + l.sparse,
                                       st));
  return launched(launch_sparse(*desc, q_sparse, k, v, kv_stride, ctx_len, kv_capacity, top_idx,
                                top_cnt, o, lse, w + l.sparse, st));
}

hs2_status hs2_decode_step_blocks(const hs2_attn_desc* desc, int block_size, const void* q,
                                  const void* q_sparse, const void* k, const void* v,
                                  int64_t kv_stride, const int32_t* ctx_len, int kv_capacity,
                                  float* scores, float* lse_full, int32_t* top_idx,
                                  int32_t* top_cnt, float* o, float* lse, void* ws,
                                  size_t ws_bytes, hs2_stream_t stream) {
  const hs2_status s =
      validate_step_blocks(desc, block_size, q, q_sparse, k, v, kv_stride, ctx_len, kv_capacity,
                           scores, lse_full, top_idx, top_cnt, o, lse, ws, ws_bytes);
  if (s != HS2_OK) return s;
  if (q_sparse == nullptr) q_sparse = q;
  (void)hipGetLastError();
  const WsLayout l = ws_layout(*desc, kv_capacity);
  char* w = static_cast<char*>(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool pf = is_prefill(*desc);
  // The same scores as hs2_full_attn_scores, then the block sums and the
  // block selection.
  hipError_t e =
      pf ? launch_prefill_scores(*desc, q, k, kv_stride, ctx_len, kv_capacity, scores, lse_full,
                                 w + l.score, false, st)
         : launch_score_decode(*desc, q, k, kv_stride, ctx_len, kv_capacity, scores, lse_full,
                               w + l.score, reinterpret_cast<uint64_t*>(w + l.sync), false, st);
  if (e != hipSuccess) return HS2_EHIP;
  e = launch_select_blocks(*desc, block_size, scores, ctx_len, kv_capacity, top_idx, top_cnt,
                           w + l.select, st);
  if (e != hipSuccess) return HS2_EHIP;
  if (pf)
    return launched(launch_prefill_sparse(*desc, q_sparse, k, v, kv_stride, ctx_len, kv_capacity,
                                          top_idx, top_cnt, o, lse, st));
  return launched(launch_sparse(*desc, q_sparse, k, v, kv_stride, ctx_len, kv_capacity, top_idx,
                                top_cnt, o, lse, w + l.sparse, st));
}

hs2_status hs2_bridge_kv_decode(const uint16_t* h, int64_t ldh, const uint16_t* w_packed,
                                int rows, int d_model, int head_dim, const int32_t* pos,
                                uint16_t* k_cache, uint16_t* v_cache, int64_t kv_stride,
                                int kv_capacity, hs2_stream_t stream) {
  const hs2_status s = validate_bridge_kv_decode(h, ldh, w_packed, rows, d_model, head_dim, pos,
                                                 k_cache, v_cache, kv_stride, kv_capacity);
  if (s != HS2_OK) return s;
  (void)hipGetLastError();
  return launched(launch_bridge_decode(h, ldh, w_packed, rows, d_model, pos, k_cache, v_cache,
                                       kv_stride, kv_capacity, static_cast<hipStream_t>(stream)));
}

hs2_status hs2_swa_attention(const hs2_attn_desc* desc, const void* q, const void* k,
                             const void* v, int64_t kv_stride, const int32_t* ctx_len,
                             int kv_capacity, void* o, hs2_dtype o_dtype, float* lse,
                             hs2_stream_t stream) {
  int o_dt;
  static_assert(sizeof(o_dt) == sizeof(o_dtype), "hs2_dtype is passed as an int");
  memcpy(&o_dt, &o_dtype, sizeof o_dt);  // any value a C caller passed
  const hs2_status s = validate_swa_attention(desc, q, k, v, kv_stride, ctx_len, kv_capacity, o,
                                              o_dt, lse);
  if (s != HS2_OK) return s;
  const hs2_attn_desc& d = *desc;
  (void)hipGetLastError();
  return launched(launch_swa(d, q, k, v, kv_stride, ctx_len, kv_capacity, o,
                             o_dtype == HS2_BF16, lse, static_cast<hipStream_t>(stream)));
}

hs2_status hs2_bridge_kv(const uint16_t* h, int64_t ldh, const uint16_t* w_k, const uint16_t* w_v,
                         uint16_t* k_out, uint16_t* v_out, int64_t ld_kv, int M, int d_model,
                         int head_dim, hs2_stream_t stream) {
  const hs2_status st =
      validate_bridge_kv(h, ldh, w_k, w_v, k_out, v_out, ld_kv, M, d_model, head_dim);
  if (st != HS2_OK) return st;
  (void)hipGetLastError();
  return launched(launch_bridge(h, ldh, nullptr, w_k, w_v, k_out, v_out, ld_kv, M, d_model,
                                static_cast<hipStream_t>(stream)));
}

hs2_status hs2_bridge_kv_packed(const uint16_t* h, int64_t ldh, const uint16_t* w_packed,
                                uint16_t* k_out, uint16_t* v_out, int64_t ld_kv, int M,
                                int d_model, int head_dim, hs2_stream_t stream) {
  const hs2_status st =
      validate_bridge_kv_packed(h, ldh, w_packed, k_out, v_out, ld_kv, M, d_model, head_dim);
  if (st != HS2_OK) return st;
  (void)hipGetLastError();
  return launched(launch_bridge(h, ldh, w_packed, nullptr, nullptr, k_out, v_out, ld_kv, M,
                                d_model, static_cast<hipStream_t>(stream)));
}

size_t hs2_bridge_packed_bytes(int d_model, int head_dim) {
  return bridge_packed_bytes(d_model, head_dim);
}

hs2_status hs2_bridge_pack_weights(const uint16_t* w_k, const uint16_t* w_v, int d_model,
                                   int head_dim, uint16_t* w_packed, hs2_stream_t stream) {
  const hs2_status st = validate_bridge_pack_weights(w_k, w_v, d_model, head_dim, w_packed);
  if (st != HS2_OK) return st;
  (void)hipGetLastError();
  return launched(launch_bridge_pack(w_k, w_v, w_packed, d_model, static_cast<hipStream_t>(stream)));
}

const char* hs2_status_string(hs2_status status) {
  switch (status) {
    case HS2_OK: return "HS2_OK: success";
    case HS2_EINVAL: return "HS2_EINVAL: null pointer, bad size or inconsistent shape";
    case HS2_EUNSUPPORTED: return "HS2_EUNSUPPORTED: valid arguments outside what the kernels implement";
    case HS2_EALIGN: return "HS2_EALIGN: pointer or stride not 16-byte aligned";
    case HS2_EWORKSPACE: return "HS2_EWORKSPACE: workspace smaller than hs2_workspace_size()";
    case HS2_EHIP: return "HS2_EHIP: the HIP runtime reported an error while enqueuing";
  }
  return "unknown hs2_status";
}

}  // extern "C"
