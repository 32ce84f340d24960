// Host-side argument checks of every libhs2 entry point: plain C++ (no HIP),
// so that they build and run on their own (the host validation tests build
// them with the address and undefined-behaviour sanitizers).  Each check
// returns HS2_OK when the entry point may enqueue, else the status that the
// entry point returns; none dereferences a device pointer or calls the HIP
// runtime.  Pointers only have to be non-null where include/hs2.h says so
// and 16-byte aligned.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "layout.h"

namespace hs2 {

constexpr int kMaxSelectCap = 1024 * kSelSlice;  // selector pools up to 4,194,304 keys
constexpr int kMaxLayers = 64;                   // sparse layers per shared selection

// The descriptor alone (shared by the attention entry points).
hs2_status check_desc(const hs2_attn_desc* d);

// hs2_workspace_size, hs2_sparse_layers_workspace_size, hs2_bridge_packed_bytes
// (0 for invalid arguments).
size_t workspace_bytes(const hs2_attn_desc* d, int kv_capacity);
size_t layers_workspace_bytes(const hs2_attn_desc* d, int n_layers);
size_t bridge_packed_bytes(int d_model, int head_dim);

hs2_status validate_full_attn_scores(const hs2_attn_desc* desc, const void* q, const void* k,
                                     const void* v, int64_t kv_stride, const int32_t* ctx_len,
                                     int kv_capacity, const float* scores, const float* o_full,
                                     const float* lse, const void* ws, size_t ws_bytes);
hs2_status validate_select_topk_window(const hs2_attn_desc* desc, const float* scores,
                                       const int32_t* ctx_len, int kv_capacity,
                                       const int32_t* top_idx, const int32_t* top_cnt,
                                       const void* ws, size_t ws_bytes);
hs2_status validate_select_topk_blocks(const hs2_attn_desc* desc, int block_size,
                                       const float* scores, const int32_t* ctx_len,
                                       int kv_capacity, const int32_t* top_idx,
                                       const int32_t* top_cnt, const void* ws, size_t ws_bytes);
hs2_status validate_sparse_attn_gather(const hs2_attn_desc* desc, const void* q, const void* k,
                                       const void* v, int64_t kv_stride, const int32_t* ctx_len,
                                       int kv_capacity, const int32_t* top_idx,
                                       const int32_t* top_cnt, const float* o, const float* lse,
                                       const void* ws, size_t ws_bytes);
hs2_status validate_sparse_attn_gather_layers(const hs2_attn_desc* desc, int n_layers,
                                              const void* q_layers, const void* k, const void* v,
                                              int64_t kv_stride, const int32_t* ctx_len,
                                              int kv_capacity, const int32_t* top_idx,
                                              const int32_t* top_cnt, const float* o_layers,
                                              const float* lse_layers, const void* ws,
                                              size_t ws_bytes);
// hs2_decode_step without its workspace (q_sparse null stands for q).
hs2_status validate_step_args(const hs2_attn_desc* desc, const void* q, const void* q_sparse,
                              const void* k, const void* v, int64_t kv_stride,
                              const int32_t* ctx_len, int kv_capacity, const float* scores,
                              const float* lse_full, const int32_t* top_idx,
                              const int32_t* top_cnt, const float* o, const float* lse);
hs2_status validate_step(const hs2_attn_desc* desc, const void* q, const void* q_sparse,
                         const void* k, const void* v, int64_t kv_stride, const int32_t* ctx_len,
                         int kv_capacity, const float* scores, const float* lse_full,
                         const int32_t* top_idx, const int32_t* top_cnt, const float* o,
                         const float* lse, const void* ws, size_t ws_bytes);
hs2_status validate_step_blocks(const hs2_attn_desc* desc, int block_size, const void* q,
                                const void* q_sparse, const void* k, const void* v,
                                int64_t kv_stride, const int32_t* ctx_len, int kv_capacity,
                                const float* scores, const float* lse_full,
                                const int32_t* top_idx, const int32_t* top_cnt, const float* o,
                                const float* lse, const void* ws, size_t ws_bytes);
// hs2_decode_step_noalloc: the step's arguments, then its workspace against
// the library's scratch size.
hs2_status validate_step_noalloc(const hs2_attn_desc* desc, const void* q, const void* q_sparse,
                                 const void* k, const void* v, int64_t kv_stride,
                                 const int32_t* ctx_len, int kv_capacity, const float* scores,
                                 const float* lse_full, const int32_t* top_idx,
                                 const int32_t* top_cnt, const float* o, const float* lse,
                                 size_t scratch_bytes);
hs2_status validate_swa_attention(const hs2_attn_desc* desc, const void* q, const void* k,
                                  const void* v, int64_t kv_stride, const int32_t* ctx_len,
                                  int kv_capacity, const void* o, int o_dtype, const float* lse);
hs2_status validate_bridge_kv(const uint16_t* h, int64_t ldh, const uint16_t* w_k,
                              const uint16_t* w_v, const uint16_t* k_out, const uint16_t* v_out,
                              int64_t ld_kv, int M, int d_model, int head_dim);
hs2_status validate_bridge_kv_packed(const uint16_t* h, int64_t ldh, const uint16_t* w_packed,
                                     const uint16_t* k_out, const uint16_t* v_out, int64_t ld_kv,
                                     int M, int d_model, int head_dim);
hs2_status validate_bridge_pack_weights(const uint16_t* w_k, const uint16_t* w_v, int d_model,
                                        int head_dim, const uint16_t* w_packed);
hs2_status validate_bridge_kv_decode(const uint16_t* h, int64_t ldh, const uint16_t* w_packed,
                                     int rows, int d_model, int head_dim, const int32_t* pos,
                                     const uint16_t* k_cache, const uint16_t* v_cache,
                                     int64_t kv_stride, int kv_capacity);

}  // namespace hs2
