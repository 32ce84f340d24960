// Sizes and the device workspace layout of libhs2: plain host C++ (no HIP),
// shared by the kernels' launchers and the host-side argument checks.
#pragma once

#include <stddef.h>
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

// Keys per workgroup of the MFMA sparse-attention kernels.
constexpr int kSegB = 128;
// Block-level selection: blocks per row.
constexpr int kMaxBlocks = 65536;
// Query rows (batch x n_q) per call: with at most kMaxSelectCap keys every
// workspace size stays far below 2^64 bytes.
constexpr int64_t kMaxQueryRows = int64_t(1) << 24;

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

// Words of the one-pass scoring kernel's barriers: a generation per sequence
// at word b, and per (sequence, workgroup) a slot of the first barrier at
// word kOpMaxWg * (1 + 2b) + c and one of the second at kOpMaxWg * (2 + 2b) + c,
// the same positions for every descriptor.
inline size_t sync_words(const hs2_attn_desc& d) {
  return (size_t)kOpMaxWg * (1 + 2 * (size_t)d.batch);
}

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

// Workgroups (segments of kSegB selected keys) of the MFMA sparse kernels.
inline int mfma_segments(const hs2_attn_desc& d) {
  const int sel_max = d.k_top + d.window;
  return sel_max > 0 ? (sel_max + kSegB - 1) / kSegB : 1;
}

// Workspace of hs2_sparse_attn_gather_layers: partial outputs and (max, sum)
// per (layer, sequence, segment, head).
inline size_t sparse_layers_ws_bytes(const hs2_attn_desc& d, int n_layers) {
  const size_t nseg = mfma_segments(d);
  const size_t rows = (size_t)n_layers * d.batch;
  return align_up(sizeof(float) * rows * nseg * d.n_heads * kHeadDim, 256) +
         align_up(sizeof(float) * 2 * rows * nseg * d.n_heads, 256);
}

}  // namespace hs2
