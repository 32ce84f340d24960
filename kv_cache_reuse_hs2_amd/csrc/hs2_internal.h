// Internal declarations shared by the libhs2 HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hs2.h"

namespace hs2 {

constexpr int kHeadDim = 128;
constexpr int kMaxHeads = 32;
constexpr int kMaxTop = 2048;
constexpr int kMaxWindow = 2048;

// Keys per workgroup of the decode scoring passes (4 waves x 8 blocks of 32).
constexpr int kScoreChunk = 1024;
// Keys per workgroup of the sparse gather kernel.
constexpr int kSparseSeg = 32;
// Top-k selection: first radix digit = top 12 bits of the orderable key.
constexpr int kSelBins = 4096;
constexpr int kSelSlice = 4096;  // pool keys per workgroup of the radix passes

// ---------------------------------------------------------------------------
// Small device helpers.

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Monotone map of an fp32 value to uint32 (larger float -> larger key); -0 is
// folded onto +0 so that equal values give equal keys.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int clamp_ctx(const int32_t* ctx_len, int b, int cap) {
  int n = ctx_len[b];
  return n < 0 ? 0 : (n > cap ? cap : n);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Workspace layout.  Every call lays its scratch out from the start of the
// caller's workspace; hs2_workspace_size() returns the maximum over calls.

struct ScoreWs {
  size_t stats_off;   // float2 [B][nchunks][32]  (max, sum) per chunk & head, base 2
  size_t lse2_off;    // float  [B][32]            per-head log2-sum-exp (+inf pad)
  size_t bytes;
};

struct SelectWs {
  size_t hist_off;    // uint32 [R][kSelBins]
  size_t ctr_off;     // uint32 [R][4]   greater count, candidate count
  size_t greater_off; // int32  [R][kMaxTop]
  size_t cand_off;    // uint2  [R][cap] (key, index)
  size_t bytes;
};

struct SparseWs {
  size_t part_off;    // float [B*n_q][nseg][H][D]  partial outputs
  size_t ml_off;      // float2 [B*n_q][nseg][H]   partial (max, sum), natural log
  size_t bytes;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Keys per workgroup of the decode scoring passes for each storage type.
inline int score_chunk_keys(hs2_dtype dt) { return dt == HS2_BF16 ? kScoreChunk : 256; }
inline int score_chunks(const hs2_attn_desc& d, int cap) {
  const int c = score_chunk_keys(d.dtype);
  return (cap + c - 1) / c;
}

inline ScoreWs score_ws(const hs2_attn_desc& d, int cap) {
  ScoreWs w{};
  size_t off = 0;
  w.stats_off = off;
  off = align_up(off + sizeof(float) * 2 * (size_t)d.batch * score_chunks(d, cap) * kMaxHeads, 256);
  w.lse2_off = off;
  off = align_up(off + sizeof(float) * (size_t)d.batch * d.n_q * kMaxHeads, 256);
  w.bytes = off;
  return w;
}

inline SelectWs select_ws(const hs2_attn_desc& d, int cap) {
  SelectWs w{};
  const size_t rows = (size_t)d.batch * (d.n_q / d.tile_q);
  size_t off = 0;
  w.hist_off = off;
  off = align_up(off + sizeof(uint32_t) * rows * kSelBins, 256);
  w.ctr_off = off;
  off = align_up(off + sizeof(uint32_t) * rows * 4, 256);
  w.greater_off = off;
  off = align_up(off + sizeof(int32_t) * rows * kMaxTop, 256);
  w.cand_off = off;
  off = align_up(off + sizeof(uint32_t) * 2 * rows * (size_t)cap, 256);
  w.bytes = off;
  return w;
}

inline int sparse_segments(const hs2_attn_desc& d) {
  return (d.k_top + d.window + kSparseSeg - 1) / kSparseSeg;
}

inline SparseWs sparse_ws(const hs2_attn_desc& d) {
  SparseWs w{};
  const size_t nq = (size_t)d.batch * d.n_q;
  const size_t nseg = sparse_segments(d) > 0 ? sparse_segments(d) : 1;
  size_t off = 0;
  w.part_off = off;
  off = align_up(off + sizeof(float) * nq * nseg * d.n_heads * kHeadDim, 256);
  w.ml_off = off;
  off = align_up(off + sizeof(float) * 2 * nq * nseg * d.n_heads, 256);
  w.bytes = off;
  return w;
}

// ---------------------------------------------------------------------------
// Kernel launchers (each returns hipGetLastError() of its launches).

hipError_t launch_score_decode(const hs2_attn_desc& d, const void* q, const void* k,
                               int64_t kv_stride, const int32_t* ctx_len, int cap,
                               float* scores, float* lse, char* ws, hipStream_t st);

hipError_t launch_select(const hs2_attn_desc& d, const float* scores, const int32_t* ctx_len,
                         int cap, int32_t* top_idx, int32_t* top_cnt, char* ws, hipStream_t st);

hipError_t launch_sparse(const hs2_attn_desc& d, const void* q, const void* k, const void* v,
                         int64_t kv_stride, const int32_t* ctx_len, int cap,
                         const int32_t* top_idx, const int32_t* top_cnt, float* o, float* lse,
                         char* ws, hipStream_t st);

}  // namespace hs2
