// Host-side argument checks of the libhs2 entry points (declared in
// validate.h).  Plain C++: no HIP runtime call and no device memory access.
#include "validate.h"

#include <math.h>
#include <string.h>

namespace hs2 {
namespace {

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// The storage type as the integer a C caller stored (any value), so that an
// out-of-range value is rejected rather than loaded as an enumerator.
int dtype_of(const hs2_attn_desc* d) {
  int v;
  static_assert(sizeof(v) == sizeof(d->dtype), "hs2_dtype is stored as an int");
  memcpy(&v, &d->dtype, sizeof v);
  return v;
}

bool finite_positive(float x) { return x > 0.f && isfinite(x); }

hs2_status check_cache(const hs2_attn_desc* d, int64_t kv_stride, int cap) {
  if (cap < 1) return HS2_EINVAL;
  if (cap > kMaxSelectCap) return HS2_EUNSUPPORTED;
  if (kv_stride < (int64_t)cap * kHeadDim) return HS2_EINVAL;
  // Keeps every row 16-byte aligned (8 bf16 or 16 fp8 elements).
  if (kv_stride % (dtype_of(d) == HS2_FP8_E4M3 ? 16 : 8) != 0) return HS2_EALIGN;
  return HS2_OK;
}

hs2_status check_ws(const hs2_attn_desc& d, int cap, const void* ws, size_t ws_bytes) {
  const size_t need = ws_layout(d, cap).bytes;
  if (ws_bytes < need) return HS2_EWORKSPACE;
  if (need > 0 && ws == nullptr) return HS2_EINVAL;
  if (misaligned(ws)) return HS2_EALIGN;
  return HS2_OK;
}

// Block-level selection: block size a power of two up to 64 dividing k_top,
// at most kMaxBlocks blocks per row (cap >= 1 checked before).
hs2_status check_block(const hs2_attn_desc* d, int block, int cap) {
  if (block < 1 || block > 64 || (block & (block - 1)) != 0) return HS2_EINVAL;
  if (d->k_top % block != 0) return HS2_EINVAL;
  if ((cap + block - 1) / block > kMaxBlocks) return HS2_EUNSUPPORTED;
  return HS2_OK;
}

// Selection inputs shared by the two selectors (after the descriptor).
hs2_status check_select(const hs2_attn_desc* desc, const float* scores, const int32_t* ctx_len,
                        int cap, const int32_t* top_idx, const int32_t* top_cnt) {
  if (scores == nullptr || ctx_len == nullptr || top_cnt == nullptr) return HS2_EINVAL;
  if (top_idx == nullptr && desc->k_top > 0) return HS2_EINVAL;
  if (cap < 1) return HS2_EINVAL;
  if (cap > kMaxSelectCap) return HS2_EUNSUPPORTED;
  return HS2_OK;
}

hs2_status check_bridge(const uint16_t* h, int64_t ldh, const uint16_t* k_out,
                        const uint16_t* v_out, int64_t ld_kv, int M, int d_model, int head_dim) {
  if (h == nullptr || k_out == nullptr || v_out == nullptr) return HS2_EINVAL;
  if (M < 1 || d_model < 1 || head_dim < 1 || ldh < d_model || ld_kv < head_dim) return HS2_EINVAL;
  if (head_dim != kHeadDim || d_model % 64 != 0) return HS2_EUNSUPPORTED;
  if (ldh % 8 != 0 || ld_kv % 8 != 0) return HS2_EALIGN;
  if (misaligned(h) || misaligned(k_out) || misaligned(v_out)) return HS2_EALIGN;
  return HS2_OK;
}

}  // namespace

hs2_status check_desc(const hs2_attn_desc* d) {
  if (d == nullptr) return HS2_EINVAL;
  if (d->batch < 1 || d->n_q < 1 || d->n_heads < 1 || d->head_dim < 1 || d->tile_q < 1)
    return HS2_EINVAL;
  if (d->k_top < 0 || d->window < 0) return HS2_EINVAL;
  if (d->n_q % d->tile_q != 0) return HS2_EINVAL;
  if (!finite_positive(d->sm_scale)) return HS2_EINVAL;
  const int dt = dtype_of(d);
  if (dt != HS2_F32 && dt != HS2_BF16 && dt != HS2_FP8_E4M3) return HS2_EINVAL;
  if (dt == HS2_FP8_E4M3 && (!finite_positive(d->k_scale) || !finite_positive(d->v_scale)))
    return HS2_EINVAL;
  if (d->head_dim != kHeadDim || d->n_heads > kMaxHeads) return HS2_EUNSUPPORTED;
  if (d->k_top > kMaxTop || d->window > kMaxWindow) return HS2_EUNSUPPORTED;
  if (d->causal != 1) return HS2_EUNSUPPORTED;
  if ((int64_t)d->batch * d->n_q > kMaxQueryRows) return HS2_EUNSUPPORTED;
  // Decode: one query per sequence.  Chunked prefill: bf16 or E4M3 K/V,
  // query tiles of a multiple of 16 queries (the kernels work on blocks of
  // 16 queries).
  const bool decode = d->n_q == 1 && d->tile_q == 1;
  const bool prefill = d->tile_q > 1 && d->tile_q % 16 == 0 && (dt == HS2_BF16 || dt == HS2_FP8_E4M3);
  if (!decode && !prefill) return HS2_EUNSUPPORTED;
  return HS2_OK;
}

size_t workspace_bytes(const hs2_attn_desc* d, int kv_capacity) {
  if (check_desc(d) != HS2_OK || kv_capacity < 1 || kv_capacity > kMaxSelectCap) return 0;
  return ws_layout(*d, kv_capacity).bytes;
}

size_t layers_workspace_bytes(const hs2_attn_desc* d, int n_layers) {
  if (check_desc(d) != HS2_OK || n_layers < 1 || n_layers > kMaxLayers) return 0;
  return sparse_layers_ws_bytes(*d, n_layers);
}

size_t bridge_packed_bytes(int d_model, int head_dim) {
  if (d_model < 64 || d_model % 64 != 0 || head_dim != kHeadDim) return 0;
  return (size_t)d_model * 2 * kHeadDim * sizeof(uint16_t);
}

hs2_status validate_full_attn_scores(const hs2_attn_desc* desc, const void* q, const void* k,
                                     const void* v, int64_t kv_stride, const int32_t* ctx_len,
                                     int kv_capacity, const float* scores, const float* o_full,
                                     const float* lse, const void* ws, size_t ws_bytes) {
  hs2_status s = check_desc(desc);
  if (s != HS2_OK) return s;
  if (q == nullptr || k == nullptr || ctx_len == nullptr || scores == nullptr) return HS2_EINVAL;
  if (o_full != nullptr && v == nullptr) return HS2_EINVAL;
  if ((s = check_cache(desc, kv_stride, kv_capacity)) != HS2_OK) return s;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(ctx_len) ||
      misaligned(scores) || misaligned(o_full) || misaligned(lse))
    return HS2_EALIGN;
  return check_ws(*desc, kv_capacity, ws, ws_bytes);
}

hs2_status validate_select_topk_window(const hs2_attn_desc* desc, const float* scores,
                                       const int32_t* ctx_len, int kv_capacity,
                                       const int32_t* top_idx, const int32_t* top_cnt,
                                       const void* ws, size_t ws_bytes) {
  hs2_status s = check_desc(desc);
  if (s != HS2_OK) return s;
  if ((s = check_select(desc, scores, ctx_len, kv_capacity, top_idx, top_cnt)) != HS2_OK)
    return s;
  if (misaligned(scores) || misaligned(ctx_len) || misaligned(top_idx) || misaligned(top_cnt))
    return HS2_EALIGN;
  return check_ws(*desc, kv_capacity, ws, ws_bytes);
}

hs2_status validate_select_topk_blocks(const hs2_attn_desc* desc, int block_size,
                                       const float* scores, const int32_t* ctx_len,
                                       int kv_capacity, const int32_t* top_idx,
                                       const int32_t* top_cnt, const void* ws, size_t ws_bytes) {
  hs2_status s = check_desc(desc);
  if (s != HS2_OK) return s;
  if ((s = check_select(desc, scores, ctx_len, kv_capacity, top_idx, top_cnt)) != HS2_OK)
    return s;
  if ((s = check_block(desc, block_size, kv_capacity)) != HS2_OK) return s;
  if (misaligned(scores) || misaligned(ctx_len) || misaligned(top_idx) || misaligned(top_cnt))
    return HS2_EALIGN;
  return check_ws(*desc, kv_capacity, ws, ws_bytes);
}

hs2_status validate_sparse_attn_gather(const hs2_attn_desc* desc, const void* q, const void* k,
                                       const void* v, int64_t kv_stride, const int32_t* ctx_len,
                                       int kv_capacity, const int32_t* top_idx,
                                       const int32_t* top_cnt, const float* o, const float* lse,
                                       const void* ws, size_t ws_bytes) {
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
  return check_ws(*desc, kv_capacity, ws, ws_bytes);
}

hs2_status validate_sparse_attn_gather_layers(const hs2_attn_desc* desc, int n_layers,
                                              const void* q_layers, const void* k, const void* v,
                                              int64_t kv_stride, const int32_t* ctx_len,
                                              int kv_capacity, const int32_t* top_idx,
                                              const int32_t* top_cnt, const float* o_layers,
                                              const float* lse_layers, const void* ws,
                                              size_t ws_bytes) {
  hs2_status s = check_desc(desc);
  if (s != HS2_OK) return s;
  if (q_layers == nullptr || k == nullptr || v == nullptr || ctx_len == nullptr ||
      top_cnt == nullptr || o_layers == nullptr)
    return HS2_EINVAL;
  if (top_idx == nullptr && desc->k_top > 0) return HS2_EINVAL;
  if (n_layers < 1) return HS2_EINVAL;
  if (n_layers > kMaxLayers || is_prefill(*desc) || dtype_of(desc) == HS2_F32)
    return HS2_EUNSUPPORTED;
  if ((s = check_cache(desc, kv_stride, kv_capacity)) != HS2_OK) return s;
  if (misaligned(q_layers) || misaligned(k) || misaligned(v) || misaligned(ctx_len) ||
      misaligned(top_idx) || misaligned(top_cnt) || misaligned(o_layers) ||
      misaligned(lse_layers) || misaligned(ws))
    return HS2_EALIGN;
  if (ws_bytes < sparse_layers_ws_bytes(*desc, n_layers)) return HS2_EWORKSPACE;
  if (ws == nullptr) return HS2_EINVAL;
  return HS2_OK;
}

hs2_status validate_step_args(const hs2_attn_desc* desc, const void* q, const void* q_sparse,
                              const void* k, const void* v, int64_t kv_stride,
                              const int32_t* ctx_len, int kv_capacity, const float* scores,
                              const float* lse_full, const int32_t* top_idx,
                              const int32_t* top_cnt, const float* o, const float* lse) {
  hs2_status s = check_desc(desc);
  if (s != HS2_OK) return s;
  if (q_sparse == nullptr) q_sparse = q;
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

hs2_status validate_step(const hs2_attn_desc* desc, const void* q, const void* q_sparse,
                         const void* k, const void* v, int64_t kv_stride, const int32_t* ctx_len,
                         int kv_capacity, const float* scores, const float* lse_full,
                         const int32_t* top_idx, const int32_t* top_cnt, const float* o,
                         const float* lse, const void* ws, size_t ws_bytes) {
  const hs2_status s = validate_step_args(desc, q, q_sparse, k, v, kv_stride, ctx_len,
                                          kv_capacity, scores, lse_full, top_idx, top_cnt, o, lse);
  if (s != HS2_OK) return s;
  return check_ws(*desc, kv_capacity, ws, ws_bytes);
}

hs2_status validate_step_blocks(const hs2_attn_desc* desc, int block_size, const void* q,
                                const void* q_sparse, const void* k, const void* v,
                                int64_t kv_stride, const int32_t* ctx_len, int kv_capacity,
                                const float* scores, const float* lse_full,
                                const int32_t* top_idx, const int32_t* top_cnt, const float* o,
                                const float* lse, const void* ws, size_t ws_bytes) {
  const hs2_status s = validate_step(desc, q, q_sparse, k, v, kv_stride, ctx_len, kv_capacity,
                                     scores, lse_full, top_idx, top_cnt, o, lse, ws, ws_bytes);
  if (s != HS2_OK) return s;
  return check_block(desc, block_size, kv_capacity);
}

hs2_status validate_step_noalloc(const hs2_attn_desc* desc, const void* q, const void* q_sparse,
                                 const void* k, const void* v, int64_t kv_stride,
                                 const int32_t* ctx_len, int kv_capacity, const float* scores,
                                 const float* lse_full, const int32_t* top_idx,
                                 const int32_t* top_cnt, const float* o, const float* lse,
                                 size_t scratch_bytes) {
  const hs2_status s = validate_step_args(desc, q, q_sparse, k, v, kv_stride, ctx_len,
                                          kv_capacity, scores, lse_full, top_idx, top_cnt, o, lse);
  if (s != HS2_OK) return s;
  return ws_layout(*desc, kv_capacity).bytes > scratch_bytes ? HS2_EWORKSPACE : HS2_OK;
}

hs2_status validate_swa_attention(const hs2_attn_desc* desc, const void* q, const void* k,
                                  const void* v, int64_t kv_stride, const int32_t* ctx_len,
                                  int kv_capacity, const void* o, int o_dtype, const float* lse) {
  if (desc == nullptr) return HS2_EINVAL;
  const hs2_attn_desc& d = *desc;
  const int dt = dtype_of(desc);
  if (d.batch < 1 || d.n_q < 1 || d.n_heads < 1 || d.head_dim < 1 || d.window < 1)
    return HS2_EINVAL;
  if (!finite_positive(d.sm_scale)) return HS2_EINVAL;
  if (dt != HS2_F32 && dt != HS2_BF16 && dt != HS2_FP8_E4M3) return HS2_EINVAL;
  if (d.head_dim != kHeadDim || d.n_heads > kMaxHeads || d.causal != 1 || dt != HS2_BF16)
    return HS2_EUNSUPPORTED;
  if (q == nullptr || k == nullptr || v == nullptr || ctx_len == nullptr || o == nullptr)
    return HS2_EINVAL;
  if (o_dtype != HS2_F32 && o_dtype != HS2_BF16) return HS2_EINVAL;
  if (kv_capacity < 1 || kv_stride < (int64_t)kv_capacity * kHeadDim) return HS2_EINVAL;
  if (kv_stride % 8 != 0) return HS2_EALIGN;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(ctx_len) || misaligned(o) ||
      misaligned(lse))
    return HS2_EALIGN;
  return HS2_OK;
}

hs2_status validate_bridge_kv(const uint16_t* h, int64_t ldh, const uint16_t* w_k,
                              const uint16_t* w_v, const uint16_t* k_out, const uint16_t* v_out,
                              int64_t ld_kv, int M, int d_model, int head_dim) {
  if (w_k == nullptr || w_v == nullptr) return HS2_EINVAL;
  const hs2_status s = check_bridge(h, ldh, k_out, v_out, ld_kv, M, d_model, head_dim);
  if (s != HS2_OK) return s;
  if (misaligned(w_k) || misaligned(w_v)) return HS2_EALIGN;
  return HS2_OK;
}

hs2_status validate_bridge_kv_packed(const uint16_t* h, int64_t ldh, const uint16_t* w_packed,
                                     const uint16_t* k_out, const uint16_t* v_out, int64_t ld_kv,
                                     int M, int d_model, int head_dim) {
  if (w_packed == nullptr) return HS2_EINVAL;
  const hs2_status s = check_bridge(h, ldh, k_out, v_out, ld_kv, M, d_model, head_dim);
  if (s != HS2_OK) return s;
  if (misaligned(w_packed)) return HS2_EALIGN;
  return HS2_OK;
}

hs2_status validate_bridge_pack_weights(const uint16_t* w_k, const uint16_t* w_v, int d_model,
                                        int head_dim, const uint16_t* w_packed) {
  if (w_k == nullptr || w_v == nullptr || w_packed == nullptr) return HS2_EINVAL;
  if (d_model < 1 || head_dim < 1) return HS2_EINVAL;
  if (head_dim != kHeadDim || d_model % 64 != 0) return HS2_EUNSUPPORTED;
  if (misaligned(w_k) || misaligned(w_v) || misaligned(w_packed)) return HS2_EALIGN;
  return HS2_OK;
}

hs2_status validate_bridge_kv_decode(const uint16_t* h, int64_t ldh, const uint16_t* w_packed,
                                     int rows, int d_model, int head_dim, const int32_t* pos,
                                     const uint16_t* k_cache, const uint16_t* v_cache,
                                     int64_t kv_stride, int kv_capacity) {
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
  return HS2_OK;
}

}  // namespace hs2
