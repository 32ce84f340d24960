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

// Decode scoring, bf16: both passes take 4,096 keys per workgroup (8 waves x
// 16 blocks of 32 keys).  fp32: one wave of 64 keys per workgroup in both
// passes (a thread per key), and the fp32 pass with the full layer's output
// works through 256-key sub-blocks.
constexpr int kP1Chunk = 4096;
constexpr int kP2Chunk = 4096;
constexpr int kF32Chunk = 64;
constexpr int kF32Sub = 256;
// Chunked prefill: keys per workgroup of the scoring passes.
constexpr int kPfSplit = 8192;
// Keys per workgroup of the sparse gather kernel.
constexpr int kSparseSeg = 32;
// Top-k selection: first radix digit = top 12 bits of the orderable key.
constexpr int kSelBins = 4096;
// Selector histograms per row: the top 12 key bits of the pool, then the next
// 12 bits of the keys in the threshold bin (built while filtering).
constexpr int kHistRow = 2 * kSelBins;
constexpr int kSelSlice = 4096;  // pool keys per workgroup of the selector passes
// One-pass decode scoring: at most this many workgroups per launch (one per CU).
constexpr int kOpMaxWg = 256;

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
// Workspace layout.  The three calls use disjoint regions (scoring, selection,
// sparse, in this order), so a selector histogram left by the scoring pass of
// the fused decode step survives until the selection reads it.

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int score_chunk1(hs2_dtype dt) { return dt == HS2_F32 ? kF32Chunk : kP1Chunk; }
inline int score_nchunks1(const hs2_attn_desc& d, int cap) {
  const int c = score_chunk1(d.dtype);
  return (cap + c - 1) / c;
}

struct ScoreWs {
  size_t stats_off;  // float2 [B][nchunks1][32]  (max, sum) per chunk & head, base 2
  size_t op_off;     // float  [kOpMaxWg][64]      one-pass kernel: (max, sum) per workgroup
  size_t lse2_off;   // float  [B][32]             per-head log2-sum-exp (fp32 path)
  size_t hist_off;   // uint32 [B][kHistRow]       selector histograms (fused step)
  size_t opart_off;  // float  [B][nchunks2][32][128] full-output partials per chunk
  size_t bytes;
};

struct SelectWs {
  size_t hist_off;    // uint32 [R][kHistRow]            (standalone selection)
  size_t cnt_off;     // uint32 [R][nslices]             entries kept per slice
  size_t meta_off;    // uint32 [R][4]                   threshold bin, keys above it
  size_t list_off;    // uint2  [R][nslices][kSelSlice]  (key, index), index order
  size_t bytes;
};

struct SparseWs {
  size_t part_off;    // float  [B*n_q][nseg][H][D]  partial outputs
  size_t ml_off;      // float2 [B*n_q][nseg][H]     partial (max, sum), natural log
  size_t bytes;
};

inline bool is_prefill(const hs2_attn_desc& d) { return d.tile_q > 1; }

struct PrefillWs {
  size_t stats_off;   // float2 [B][nsplit][n_q][32]
  size_t colsum_off;  // float  [B][n_q/16][cap]
  size_t hist_off;    // uint32 [B][tiles][kHistRow]
  size_t bytes;
};

inline PrefillWs prefill_ws(const hs2_attn_desc& d, int cap) {
  PrefillWs w{};
  const size_t nsplit = (cap + kPfSplit - 1) / kPfSplit;
  size_t off = 0;
  w.stats_off = off;
  off = align_up(off + sizeof(float) * 2 * (size_t)d.batch * nsplit * d.n_q * 32, 256);
  w.colsum_off = off;
  off = align_up(off + sizeof(float) * (size_t)d.batch * (d.n_q / 16) * cap, 256);
  w.hist_off = off;
  off = align_up(off + sizeof(uint32_t) * (size_t)d.batch * (d.n_q / d.tile_q) * kHistRow, 256);
  w.bytes = off;
  return w;
}

inline ScoreWs score_ws(const hs2_attn_desc& d, int cap) {
  ScoreWs w{};
  size_t off = 0;
  w.stats_off = off;
  off = align_up(off + sizeof(float) * 2 * (size_t)d.batch * score_nchunks1(d, cap) * kMaxHeads, 256);
  w.op_off = off;
  off = align_up(off + sizeof(float) * kOpMaxWg * 64, 256);
  w.lse2_off = off;
  off = align_up(off + sizeof(float) * (size_t)d.batch * d.n_q * kMaxHeads, 256);
  w.hist_off = off;
  off = align_up(off + sizeof(uint32_t) * (size_t)d.batch * kHistRow, 256);
  w.opart_off = off;
  off = align_up(off + sizeof(float) * (size_t)d.batch * ((cap + kP2Chunk - 1) / kP2Chunk) *
                           kMaxHeads * kHeadDim, 256);
  w.bytes = off;
  return w;
}

inline int select_slices(int cap) { return (cap + kSelSlice - 1) / kSelSlice; }

inline SelectWs select_ws(const hs2_attn_desc& d, int cap) {
  SelectWs w{};
  const size_t rows = (size_t)d.batch * (d.n_q / d.tile_q);
  const size_t ns = select_slices(cap);
  size_t off = 0;
  w.hist_off = off;
  off = align_up(off + sizeof(uint32_t) * rows * kHistRow, 256);
  w.cnt_off = off;
  off = align_up(off + sizeof(uint32_t) * rows * ns, 256);
  w.meta_off = off;
  off = align_up(off + sizeof(uint32_t) * rows * 4, 256);
  w.list_off = off;
  off = align_up(off + sizeof(uint32_t) * 2 * rows * ns * kSelSlice, 256);
  w.bytes = off;
  return w;
}

inline int sparse_segments(const hs2_attn_desc& d) {
  const int n = (d.k_top + d.window + kSparseSeg - 1) / kSparseSeg;
  return n > 0 ? n : 1;
}

inline SparseWs sparse_ws(const hs2_attn_desc& d) {
  SparseWs w{};
  const size_t nq = (size_t)d.batch * d.n_q;
  const size_t nseg = sparse_segments(d);
  size_t off = 0;
  w.part_off = off;
  off = align_up(off + sizeof(float) * nq * nseg * d.n_heads * kHeadDim, 256);
  w.ml_off = off;
  off = align_up(off + sizeof(float) * 2 * nq * nseg * d.n_heads, 256);
  w.bytes = off;
  return w;
}

// Words of the one-pass scoring kernel's barrier: a generation per sequence at
// word b and a slot per (sequence, workgroup) at word kOpMaxWg * (1 + b) + c,
// the same positions for every descriptor.
inline size_t sync_words(const hs2_attn_desc& d) { return (size_t)kOpMaxWg * (1 + d.batch); }

// Offsets of the regions inside the caller's workspace: the barrier words at
// offset 0 (so that they keep their place whatever the descriptor), then
// scoring, selection and sparse.
struct WsLayout {
  size_t sync, score, select, sparse, bytes;
};

inline WsLayout ws_layout(const hs2_attn_desc& d, int cap) {
  WsLayout l{};
  l.sync = 0;
  l.score = align_up(sizeof(uint64_t) * sync_words(d), 256);
  l.select = align_up(l.score + (is_prefill(d) ? prefill_ws(d, cap).bytes : score_ws(d, cap).bytes), 256);
  l.sparse = align_up(l.select + select_ws(d, cap).bytes, 256);
  l.bytes = align_up(l.sparse + sparse_ws(d).bytes, 256);
  return l;
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

// with_hist: also build the selector histogram of the pool scores in the
// scoring region (MFMA paths only).  sync: the barrier words of the workspace
// (ws_layout().sync); bf16 and E4M3 K take the one-pass kernel when the batch
// fits the device, two passes otherwise.
hipError_t launch_score_decode(const hs2_attn_desc& d, const void* q, const void* k,
                               int64_t kv_stride, const int32_t* ctx_len, int cap,
                               float* scores, float* lse, char* ws, uint64_t* sync,
                               bool with_hist, hipStream_t st);

// One-pass decode scoring (bf16 or E4M3 K): workgroups per sequence and keys
// per workgroup for a device of n_cu CUs; false when the batch does not fit.
bool onepass_plan(const hs2_attn_desc& d, int cap, int n_cu, int* nwg, int* chunk);
hipError_t launch_score_onepass(const hs2_attn_desc& d, const void* q, const void* k,
                                int64_t kv_stride, const int32_t* ctx_len, int cap, int nwg,
                                int chunk, float c2, float* stats, uint64_t* sync, float* scores,
                                float* lse, uint32_t* hist, hipStream_t st);
// Compute units of the current device (cached per device).
int device_cu_count();

// Host-side checks of hs2_decode_step's arguments other than the workspace.
hs2_status check_step_args(const hs2_attn_desc* desc, const void* q, const void* q_sparse,
                           const void* k, const void* v, int64_t kv_stride,
                           const int32_t* ctx_len, int kv_capacity, const float* scores,
                           const float* lse_full, const int32_t* top_idx,
                           const int32_t* top_cnt, const float* o, const float* lse);

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
constexpr int kMaxBlocks = 65536;  // blocks per row
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
size_t sparse_layers_ws_bytes(const hs2_attn_desc& d, int n_layers);
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
