// Internal declarations shared by the libhs2 HIP sources (gfx950 only); the
// sizes and the workspace layout are in layout.h (host-only C++).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hs2.h"
#include "layout.h"

namespace hs2 {

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

// Sums over the two halves of a wave for two values at once, on the VALU
// (v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second) rather than through the LDS crossbar: lane l < 32
// gets a[l] + a[l + 32], lane l >= 32 gets b[l - 32] + b[l].  Each sum adds the
// lower half's value to the upper half's, as a single-value reduction would.
__device__ __forceinline__ float half_sums2(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Orders one wave's LDS writes before its later LDS reads by other lanes (and
// those reads before later writes).  The hardware keeps a wave's LDS accesses
// in order; the fences only stop the compiler from moving them.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Buffer resource over `bytes` bytes at p: buffer loads past the end return
// zero and stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
// Cache policy of buffer accesses to data that other workgroups of the same
// launch write or read (sc1: coherent at device scope, across the XCDs' L2s).
constexpr int kSc1 = 16;

// Bytes per stored K/V element: E4M3 caches hold one byte per element, the
// bf16 kernels two.
template <bool kFp8>
constexpr int kv_elem_bytes() {
  return kFp8 ? 1 : 2;
}

// Eight OCP E4M3 bytes (two little-endian words, lowest byte first) as eight
// bf16 values in the same order.  Every E4M3 value, subnormals included, is
// exact in bf16 (3 mantissa bits, exponents 2^-9 .. 2^8), so nothing rounds.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return r;
}

// Head dimensions that lane half hh (lane / 32) feeds to step e (0..7) of a
// 128-deep contraction on v_mfma_f32_32x32x16_bf16: eight consecutive dims
// starting at the returned one.  A dot product does not depend on the order
// of its terms, so both operands only have to agree.  bf16 rows are read as
// sixteen 16-byte pieces, piece 2e + hh feeding step e; E4M3 rows (128 bytes)
// as eight 16-byte pieces, piece 2i + hh (dims 32i + 16hh .. +16) feeding
// steps 2i and 2i + 1.  Either way the two lane halves read neighbouring
// pieces of a row in the same load instruction.
template <bool kFp8>
__device__ __forceinline__ int step_dim(int e, int hh) {
  return kFp8 ? 32 * (e >> 1) + 16 * hh + 8 * (e & 1) : 16 * e + 8 * hh;
}

// ---------------------------------------------------------------------------
// Kernel launchers (each returns hipGetLastError() of its launches).  `ws`
// points at the launcher's own region.

// Decode scoring with the full layer's own output (MFMA paths): the
// importance as launch_score_decode writes it (to within rounding) and
// o_full[b][h][:] = sum_j p_hj v_j, also streaming V.
hipError_t launch_score_full(const hs2_attn_desc& d, const void* q, const void* k, const void* v,
                             int64_t kv_stride, const int32_t* ctx_len, int cap, float* scores,
                             float* o_full, float* lse, char* ws, hipStream_t st);

// Piece sums of the pool scores for the block-level selector: out[r][m] =
// fp64 sum of the scores of keys [m*piece, (m+1)*piece) of row r (keys past
// the pool count 0), row stride `stride` doubles.
struct BlockPieces {
  double* out;
  int piece;   // min(block, 32)
  int stride;  // blk_stride(cap, piece)
};

// The selector's candidate filter as the one-pass scoring kernel runs it in
// the fused decode step: the selection region's slice counts, per-row
// metadata and candidate lists (select_ws), and the budget.
struct FilterArgs {
  uint32_t* cnt;
  uint32_t* meta;
  uint2* list;
  int nslices;
  int k_top;
};

// with_hist: also build the selector histogram of the pool scores in the
// scoring region (MFMA paths only).  sync: the barrier words of the workspace
// (ws_layout().sync); bf16 and E4M3 K take the one-pass kernel when the batch
// fits the device, two passes otherwise.  filt (with with_hist): the one-pass
// kernel also runs the selector's candidate filter, and *filtered says
// whether it did (false: the two-pass kernels ran; the filter is the
// caller's).
hipError_t launch_score_decode(const hs2_attn_desc& d, const void* q, const void* k,
                               int64_t kv_stride, const int32_t* ctx_len, int cap,
                               float* scores, float* lse, char* ws, uint64_t* sync,
                               bool with_hist, hipStream_t st, const FilterArgs* filt = nullptr,
                               bool* filtered = nullptr);

// One-pass decode scoring (bf16 or E4M3 K): workgroups per sequence and keys
// per workgroup for a device of n_cu CUs; false when the batch does not fit.
// With filt and hist, the kernel builds the histogram and runs the filter.
bool onepass_plan(const hs2_attn_desc& d, int cap, int n_cu, int* nwg, int* chunk);
hipError_t launch_score_onepass(const hs2_attn_desc& d, const void* q, const void* k,
                                int64_t kv_stride, const int32_t* ctx_len, int cap, int nwg,
                                int chunk, float c2, float* stats, uint64_t* sync, float* scores,
                                float* lse, uint32_t* hist, const FilterArgs* filt,
                                hipStream_t st);
// Compute units of the current device (cached per device).
int device_cu_count();

// hist: a ready histogram of the pool scores (from launch_score_decode with
// with_hist), or null to build one.  final_stage false: stop after the
// candidate filter (launch_decode_tail finishes the selection).
hipError_t launch_select(const hs2_attn_desc& d, const float* scores, const int32_t* ctx_len,
                         int cap, int32_t* top_idx, int32_t* top_cnt, char* ws,
                         uint32_t* hist, bool final_stage, hipStream_t st);

// Sliding-window attention (the self-decoder's SWA layers), bf16, any n_q:
// query i at N - n_q + i attends to its last d.window keys; o in bf16 or fp32.
hipError_t launch_swa(const hs2_attn_desc& d, const void* q, const void* k, const void* v,
                      int64_t kv_stride, const int32_t* ctx_len, int cap, void* o,
                      bool bf16_out, float* lse, hipStream_t st);

// Block-level selection (blocks of `block` tokens, a power of two <= 64):
// piece sums (pieces of min(block, 32) keys) in the selection region's list
// area, then one workgroup per row; writes top_idx/top_cnt like
// launch_select.
int blk_stride(int cap, int piece);
BlockPieces block_pieces(const hs2_attn_desc& d, int block, int cap, char* sel_ws);
hipError_t launch_select_blocks(const hs2_attn_desc& d, int block, const float* scores,
                                const int32_t* ctx_len, int cap, int32_t* top_idx,
                                int32_t* top_cnt, char* ws, hipStream_t st);

// Chunked prefill (tile_q > 1, bf16): scoring over query tiles and sparse
// attention of the tiles' queries.
// Prefill: the full layer's own output (after launch_prefill_scores, whose
// statistics it reads from the workspace), fp32 [B][n_q][H][128].
hipError_t launch_prefill_out(const hs2_attn_desc& d, const void* q, const void* k,
                              const void* v, int64_t kv_stride, const int32_t* ctx_len, int cap,
                              float* o_full, char* ws, hipStream_t st);

hipError_t launch_prefill_scores(const hs2_attn_desc& d, const void* q, const void* k,
                                 int64_t kv_stride, const int32_t* ctx_len, int cap,
                                 float* scores, float* lse, char* ws, bool with_hist,
                                 hipStream_t st);
hipError_t launch_prefill_sparse(const hs2_attn_desc& d, const void* q, const void* k,
                                 const void* v, int64_t kv_stride, const int32_t* ctx_len,
                                 int cap, const int32_t* top_idx, const int32_t* top_cnt,
                                 float* o, float* lse, hipStream_t st);

hipError_t launch_sparse(const hs2_attn_desc& d, const void* q, const void* k, const void* v,
                         int64_t kv_stride, const int32_t* ctx_len, int cap,
                         const int32_t* top_idx, const int32_t* top_cnt, float* o, float* lse,
                         char* ws, hipStream_t st);

// Several sparse layers sharing one selection (bf16 decode): each selected
// K/V row is gathered once for all n_layers queries; q_layers, o_layers and
// lse_layers are [n_layers][B][H][D] / [n_layers][B][H].
hipError_t launch_sparse_layers(const hs2_attn_desc& d, int n_layers, const void* q_layers,
                                const void* k, const void* v, int64_t kv_stride,
                                const int32_t* ctx_len, int cap, const int32_t* top_idx,
                                const int32_t* top_cnt, float* o_layers, float* lse_layers,
                                char* ws, hipStream_t st);

// bf16 decode after launch_select(final_stage = false): the final selection
// (to top_idx/top_cnt) and the sparse layer in one pass over the candidate
// lists of sel_ws, then the merge of the partials; same results as
// launch_select's final stage followed by launch_sparse.
hipError_t launch_decode_tail(const hs2_attn_desc& d, const void* q, const void* k, const void* v,
                              int64_t kv_stride, const int32_t* ctx_len, int cap,
                              const uint32_t* hist, const char* sel_ws, int32_t* top_idx,
                              int32_t* top_cnt, float* o, float* lse, char* sparse_ws,
                              hipStream_t st);

}  // namespace hs2
