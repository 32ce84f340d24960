// C ABI entry points of libhs2: host-side validation, then kernel dispatch.
// Every argument check happens before the first enqueue, so a call that
// returns an error has enqueued nothing.
#include <math.h>

#include "hs2_internal.h"

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

constexpr int kMaxSelectCap = 1024 * kSelSlice;  // selector pools up to 4,194,304 keys
constexpr int kMaxLayers = 64;                   // sparse layers per shared selection

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

hs2_status check_desc(const hs2_attn_desc* d) {
  if (d == nullptr) return HS2_EINVAL;
  if (d->batch < 1 || d->n_q < 1 || d->n_heads < 1 || d->head_dim < 1 || d->tile_q < 1)
    return HS2_EINVAL;
  if (d->k_top < 0 || d->window < 0) return HS2_EINVAL;
  if (d->n_q % d->tile_q != 0) return HS2_EINVAL;
  if (!(d->sm_scale > 0.f) || !isfinite(d->sm_scale)) return HS2_EINVAL;
  if (d->dtype != HS2_F32 && d->dtype != HS2_BF16 && d->dtype != HS2_FP8_E4M3) return HS2_EINVAL;
  if (d->dtype == HS2_FP8_E4M3 && (!(d->k_scale > 0.f) || !isfinite(d->k_scale) ||
                                   !(d->v_scale > 0.f) || !isfinite(d->v_scale)))
    return HS2_EINVAL;
  if (d->head_dim != kHeadDim || d->n_heads > kMaxHeads) return HS2_EUNSUPPORTED;
  if (d->k_top > kMaxTop || d->window > kMaxWindow) return HS2_EUNSUPPORTED;
  if (d->causal != 1) return HS2_EUNSUPPORTED;
  // Decode: one query per sequence.  Chunked prefill: bf16, query tiles of a
  // multiple of 16 queries (the kernels work on blocks of 16 queries).
  const bool decode = d->n_q == 1 && d->tile_q == 1;
  const bool prefill = d->tile_q > 1 && d->tile_q % 16 == 0 && d->dtype == HS2_BF16;
  if (!decode && !prefill) return HS2_EUNSUPPORTED;
  return HS2_OK;
}

hs2_status check_cache(const hs2_attn_desc* d, int64_t kv_stride, int cap) {
  if (cap < 1) return HS2_EINVAL;
  if (cap > kMaxSelectCap) return HS2_EUNSUPPORTED;
  if (kv_stride < (int64_t)cap * kHeadDim) return HS2_EINVAL;
  // Keeps every row 16-byte aligned (8 bf16 or 16 fp8 elements).
  if (kv_stride % (d->dtype == HS2_FP8_E4M3 ? 16 : 8) != 0) return HS2_EALIGN;
  (void)d;
  return HS2_OK;
}

size_t needed_ws(const hs2_attn_desc& d, int cap) { return ws_layout(d, cap).bytes; }

hs2_status check_ws(const hs2_attn_desc& d, int cap, const void* ws, size_t ws_bytes) {
  const size_t need = needed_ws(d, cap);
  if (ws_bytes < need) return HS2_EWORKSPACE;
  if (need > 0 && ws == nullptr) return HS2_EINVAL;
  if (misaligned(ws)) return HS2_EALIGN;
  return HS2_OK;
}

hs2_status launched(hipError_t e) { return e == hipSuccess ? HS2_OK : HS2_EHIP; }

// Block-level selection: block size a power of two up to 64 dividing k_top,
// at most kMaxBlocks blocks per row (cap >= 1 checked before).
hs2_status check_block(const hs2_attn_desc* d, int block, int cap) {
  if (block < 1 || block > 64 || (block & (block - 1)) != 0) return HS2_EINVAL;
  if (d->k_top % block != 0) return HS2_EINVAL;
  if ((cap + block - 1) / block > kMaxBlocks) return HS2_EUNSUPPORTED;
  return HS2_OK;
}

// Arguments of a whole step (hs2_decode_step and its block-level variant).
hs2_status check_step(const hs2_attn_desc* desc, const void* q, const void* q_sparse,
                      const void* k, const void* v, int64_t kv_stride, const int32_t* ctx_len,
                      int kv_capacity, const float* scores, const float* lse_full,
                      const int32_t* top_idx, const int32_t* top_cnt, const float* o,
                      const float* lse, const void* ws, size_t ws_bytes) {
  const hs2_status s = check_step_args(desc, q, q_sparse, k, v, kv_stride, ctx_len, kv_capacity,
                                       scores, lse_full, top_idx, top_cnt, o, lse);
  if (s != HS2_OK) return s;
  return check_ws(*desc, kv_capacity, ws, ws_bytes);
}

}  // namespace

hs2_status check_step_args(const hs2_attn_desc* desc, const void* q, const void* q_sparse,
                           const void* k, const void* v, int64_t kv_stride,
                           const int32_t* ctx_len, int kv_capacity, const float* scores,
                           const float* lse_full, const int32_t* top_idx,
                           const int32_t* top_cnt, const float* o, const float* lse) {
  hs2_status s = check_desc(desc);
  if (s != HS2_OK) return s;
  if (q == nullptr || k == nullptr || v == nullptr || ctx_len == nullptr || scores == nullptr ||
      top_cnt == nullptr || o == nullptr)
    return HS2_EINVAL;
  if (top_idx == nullptr && desc->k_top > 0) return HS2_EINVAL;
  if ((s = check_cache(desc, kv_stride, kv_capacity)) != HS2_OK) return s;
  if (misaligned(q) || misaligned(q_sparse) || misaligned(k) || misaligned(v) ||
      misaligned(ctx_len) || misaligned(scores) || misaligned(lse_full) || misaligned(top_idx) ||
      misaligned(top_cnt) || misaligned(o) || misaligned(lse))
    return HS2_EALIGN;
  return HS2_OK;
}

namespace {

hs2_status check_bridge(const uint16_t* h, int64_t ldh, uint16_t* k_out, uint16_t* v_out,
                        int64_t ld_kv, int M, int d_model, int head_dim) {
  if (h == nullptr || k_out == nullptr || v_out == nullptr) return HS2_EINVAL;
  if (M < 1 || d_model < 1 || head_dim < 1 || ldh < d_model || ld_kv < head_dim) return HS2_EINVAL;
  if (head_dim != kHeadDim || d_model % 64 != 0) return HS2_EUNSUPPORTED;
  if (ldh % 8 != 0 || ld_kv % 8 != 0) return HS2_EALIGN;
  if (misaligned(h) || misaligned(k_out) || misaligned(v_out)) return HS2_EALIGN;
  return HS2_OK;
}

}  // namespace
}  // namespace hs2

using namespace hs2;

extern "C" {

size_t hs2_workspace_size(const hs2_attn_desc* desc, int kv_capacity) {
  if (check_desc(desc) != HS2_OK || kv_capacity < 1 || kv_capacity > kMaxSelectCap) return 0;
  return needed_ws(*desc, kv_capacity);
}

hs2_status hs2_full_attn_scores(const hs2_attn_desc* desc, const void* q, const void* k,
                                const void* v, int64_t kv_stride, const int32_t* ctx_len,
                                int kv_capacity, float* scores, float* o_full, float* lse,
                                void* ws, size_t ws_bytes, hs2_stream_t stream) {
  hs2_status s = check_desc(desc);
  if (s != HS2_OK) return s;
  if (q == nullptr || k == nullptr || ctx_len == nullptr || scores == nullptr) return HS2_EINVAL;
  if (o_full != nullptr && v == nullptr) return HS2_EINVAL;
  if ((s = check_cache(desc, kv_stride, kv_capacity)) != HS2_OK) return s;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(ctx_len) ||
      misaligned(scores) || misaligned(o_full) || misaligned(lse))
    return HS2_EALIGN;
  if ((s = check_ws(*desc, kv_capacity, ws, ws_bytes)) != HS2_OK) return s;
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
  hs2_status s = check_desc(desc);
  if (s != HS2_OK) return s;
  if (scores == nullptr || ctx_len == nullptr || top_cnt == nullptr) return HS2_EINVAL;
  if (top_idx == nullptr && desc->k_top > 0) return HS2_EINVAL;
  if (kv_capacity < 1) return HS2_EINVAL;
  if (kv_capacity > kMaxSelectCap) return HS2_EUNSUPPORTED;
  if (misaligned(scores) || misaligned(ctx_len) || misaligned(top_idx) || misaligned(top_cnt))
    return HS2_EALIGN;
  if ((s = check_ws(*desc, kv_capacity, ws, ws_bytes)) != HS2_OK) return s;
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
  hs2_status s = check_desc(desc);
  if (s != HS2_OK) return s;
  if (scores == nullptr || ctx_len == nullptr || top_cnt == nullptr) return HS2_EINVAL;
  if (top_idx == nullptr && desc->k_top > 0) return HS2_EINVAL;
  if (kv_capacity < 1) return HS2_EINVAL;
  if (kv_capacity > kMaxSelectCap) return HS2_EUNSUPPORTED;
  if ((s = check_block(desc, block_size, kv_capacity)) != HS2_OK) return s;
  if (misaligned(scores) || misaligned(ctx_len) || misaligned(top_idx) || misaligned(top_cnt))
    return HS2_EALIGN;
  if ((s = check_ws(*desc, kv_capacity, ws, ws_bytes)) != HS2_OK) return s;
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
  hs2_status s = check_desc(desc);
  if (s != HS2_OK) return s;
  if (q == nullptr || k == nullptr || v == nullptr || ctx_len == nullptr || top_cnt == nullptr ||
      o == nullptr)
    return HS2_EINVAL;
  if (top_idx == nullptr && desc->k_top > 0) return HS2_EINVAL;
  if ((s = check_cache(desc, kv_stride, kv_capacity)) != HS2_OK) return s;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(ctx_len) ||
      misaligned(top_idx) || misaligned(top_cnt) || misaligned(o) || misaligned(lse))
    return HS2_EALIGN;
  if ((s = check_ws(*desc, kv_capacity, ws, ws_bytes)) != HS2_OK) return s;
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
  if (check_desc(desc) != HS2_OK || n_layers < 1 || n_layers > kMaxLayers) return 0;
  return sparse_layers_ws_bytes(*desc, n_layers);
}

hs2_status hs2_sparse_attn_gather_layers(const hs2_attn_desc* desc, int n_layers,
                                         const void* q_layers, const void* k, const void* v,
                                         int64_t kv_stride, const int32_t* ctx_len,
                                         int kv_capacity, const int32_t* top_idx,
                                         const int32_t* top_cnt, float* o_layers,
                                         float* lse_layers, void* ws, size_t ws_bytes,
                                         hs2_stream_t stream) {
  hs2_status s = check_desc(desc);
  if (s != HS2_OK) return s;
  if (q_layers == nullptr || k == nullptr || v == nullptr || ctx_len == nullptr ||
      top_cnt == nullptr || o_layers == nullptr)
    return HS2_EINVAL;
  if (top_idx == nullptr && desc->k_top > 0) return HS2_EINVAL;
  if (n_layers < 1) return HS2_EINVAL;
  if (n_layers > kMaxLayers || is_prefill(*desc) || desc->dtype == HS2_F32)
    return HS2_EUNSUPPORTED;
  if ((s = check_cache(desc, kv_stride, kv_capacity)) != HS2_OK) return s;
  if (misaligned(q_layers) || misaligned(k) || misaligned(v) || misaligned(ctx_len) ||
      misaligned(top_idx) || misaligned(top_cnt) || misaligned(o_layers) ||
      misaligned(lse_layers) || misaligned(ws))
    return HS2_EALIGN;
  if (ws_bytes < sparse_layers_ws_bytes(*desc, n_layers)) return HS2_EWORKSPACE;
  if (ws == nullptr) return HS2_EINVAL;
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
  if (q_sparse == nullptr) q_sparse = q;
  hs2_status s = check_step(desc, q, q_sparse, k, v, kv_stride, ctx_len, kv_capacity, scores,
                            lse_full, top_idx, top_cnt, o, lse, ws, ws_bytes);
  if (s != HS2_OK) return s;
  (void)hipGetLastError();
  const WsLayout l = ws_layout(*desc, kv_capacity);
  char* w = static_cast<char*>(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // bf16 and E4M3: the scoring pass also builds the selector's histogram.
  const bool fuse = desc->dtype != HS2_F32;
  const bool pf = is_prefill(*desc);
  hipError_t e =
      pf ? launch_prefill_scores(*desc, q, k, kv_stride, ctx_len, kv_capacity, scores, lse_full,
                                 w + l.score, fuse, st)
         : launch_score_decode(*desc, q, k, kv_stride, ctx_len, kv_capacity, scores, lse_full,
                               w + l.score, reinterpret_cast<uint64_t*>(w + l.sync), fuse, st);
  if (e != hipSuccess) return HS2_EHIP;
  const size_t hist_off = pf ? prefill_ws(*desc, kv_capacity).hist_off
                             : score_ws(*desc, kv_capacity).hist_off;
  uint32_t* hist = fuse ? reinterpret_cast<uint32_t*>(w + l.score + hist_off) : nullptr;
  // MFMA decode: the final selection runs inside the sparse layer's kernel.
  const bool tail = fuse && !pf;
  e = launch_select(*desc, scores, ctx_len, kv_capacity, top_idx, top_cnt, w + l.select, hist,
                    !tail, st);
  if (e != hipSuccess) return HS2_EHIP;
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
  if (q_sparse == nullptr) q_sparse = q;
  hs2_status s = check_step(desc, q, q_sparse, k, v, kv_stride, ctx_len, kv_capacity, scores,
                            lse_full, top_idx, top_cnt, o, lse, ws, ws_bytes);
  if (s != HS2_OK) return s;
  if ((s = check_block(desc, block_size, kv_capacity)) != HS2_OK) return s;
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
  if (h == nullptr || w_packed == nullptr || pos == nullptr || k_cache == nullptr ||
      v_cache == nullptr)
    return HS2_EINVAL;
  if (rows < 1 || d_model < 1 || head_dim < 1 || ldh < d_model || kv_capacity < 1)
    return HS2_EINVAL;
  if (head_dim != kHeadDim || d_model % 64 != 0) return HS2_EUNSUPPORTED;
  if (kv_stride < (int64_t)kv_capacity * kHeadDim) return HS2_EINVAL;
  if (ldh % 8 != 0 || kv_stride % 8 != 0) return HS2_EALIGN;
  if (misaligned(h) || misaligned(w_packed) || misaligned(pos) || misaligned(k_cache) ||
      misaligned(v_cache))
    return HS2_EALIGN;
  (void)hipGetLastError();
  return launched(launch_bridge_decode(h, ldh, w_packed, rows, d_model, pos, k_cache, v_cache,
                                       kv_stride, kv_capacity, static_cast<hipStream_t>(stream)));
}

hs2_status hs2_swa_attention(const hs2_attn_desc* desc, const void* q, const void* k,
                             const void* v, int64_t kv_stride, const int32_t* ctx_len,
                             int kv_capacity, void* o, hs2_dtype o_dtype, float* lse,
                             hs2_stream_t stream) {
  if (desc == nullptr) return HS2_EINVAL;
  const hs2_attn_desc& d = *desc;
  if (d.batch < 1 || d.n_q < 1 || d.n_heads < 1 || d.head_dim < 1 || d.window < 1)
    return HS2_EINVAL;
  if (!(d.sm_scale > 0.f) || !isfinite(d.sm_scale)) return HS2_EINVAL;
  if (d.dtype != HS2_F32 && d.dtype != HS2_BF16 && d.dtype != HS2_FP8_E4M3) return HS2_EINVAL;
  if (d.head_dim != kHeadDim || d.n_heads > kMaxHeads || d.causal != 1 || d.dtype != HS2_BF16)
    return HS2_EUNSUPPORTED;
  if (q == nullptr || k == nullptr || v == nullptr || ctx_len == nullptr || o == nullptr)
    return HS2_EINVAL;
  if (o_dtype != HS2_F32 && o_dtype != HS2_BF16) return HS2_EINVAL;
  if (kv_capacity < 1 || kv_stride < (int64_t)kv_capacity * kHeadDim) return HS2_EINVAL;
  if (kv_stride % 8 != 0) return HS2_EALIGN;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(ctx_len) || misaligned(o) ||
      misaligned(lse))
    return HS2_EALIGN;
  (void)hipGetLastError();
  return launched(launch_swa(d, q, k, v, kv_stride, ctx_len, kv_capacity, o,
                             o_dtype == HS2_BF16, lse, static_cast<hipStream_t>(stream)));
}

hs2_status hs2_bridge_kv(const uint16_t* h, int64_t ldh, const uint16_t* w_k, const uint16_t* w_v,
                         uint16_t* k_out, uint16_t* v_out, int64_t ld_kv, int M, int d_model,
                         int head_dim, hs2_stream_t stream) {
  if (w_k == nullptr || w_v == nullptr) return HS2_EINVAL;
  const hs2_status st = check_bridge(h, ldh, k_out, v_out, ld_kv, M, d_model, head_dim);
  if (st != HS2_OK) return st;
  if (misaligned(w_k) || misaligned(w_v)) return HS2_EALIGN;
  (void)hipGetLastError();
  return launched(launch_bridge(h, ldh, nullptr, w_k, w_v, k_out, v_out, ld_kv, M, d_model,
                                static_cast<hipStream_t>(stream)));
}

hs2_status hs2_bridge_kv_packed(const uint16_t* h, int64_t ldh, const uint16_t* w_packed,
                                uint16_t* k_out, uint16_t* v_out, int64_t ld_kv, int M,
                                int d_model, int head_dim, hs2_stream_t stream) {
  if (w_packed == nullptr) return HS2_EINVAL;
  const hs2_status st = check_bridge(h, ldh, k_out, v_out, ld_kv, M, d_model, head_dim);
  if (st != HS2_OK) return st;
  if (misaligned(w_packed)) return HS2_EALIGN;
  (void)hipGetLastError();
  return launched(launch_bridge(h, ldh, w_packed, nullptr, nullptr, k_out, v_out, ld_kv, M,
                                d_model, static_cast<hipStream_t>(stream)));
}

size_t hs2_bridge_packed_bytes(int d_model, int head_dim) {
  if (d_model < 64 || d_model % 64 != 0 || head_dim != kHeadDim) return 0;
  return (size_t)d_model * 2 * kHeadDim * sizeof(uint16_t);
}

hs2_status hs2_bridge_pack_weights(const uint16_t* w_k, const uint16_t* w_v, int d_model,
                                   int head_dim, uint16_t* w_packed, hs2_stream_t stream) {
  if (w_k == nullptr || w_v == nullptr || w_packed == nullptr) return HS2_EINVAL;
  if (d_model < 1 || head_dim < 1) return HS2_EINVAL;
  if (head_dim != kHeadDim || d_model % 64 != 0) return HS2_EUNSUPPORTED;
  if (misaligned(w_k) || misaligned(w_v) || misaligned(w_packed)) return HS2_EALIGN;
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
