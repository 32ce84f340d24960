// Token-level top-k selection with a forced recent window.
//
// HySparse2 gives its sparse layers 1,024 individual tokens chosen from the
// whole context plus the 128 most recent tokens, which are always included
// ("HySparse2: How Xiaomi Split the Transformer to Fix Agent Prefill Costs",
// section "KV Reuse and Token-Level Sparse Selection"; "HySparse2: Hybrid
// Sparse Attention with Two-Level KV Sharing", bullet "KV Reuse
// refinements").  Here the window keys are kept out of the top-k pool, the
// pool of a group whose first query sits at P0 being [0, P0 - window + 1),
// and ties go to the lower index.  The window is implied by each query's
// position and never stored.
//
// Exact radix selection on the orderable uint32 image of the fp32 score:
//   sel_init + sel_hist: per-row histogram of the top 12 bits (LDS per
//       workgroup, merged with integer atomics, so the counts do not depend
//       on scheduling).  The fused decode step gets this histogram from the
//       scoring pass instead.
//   sel_filter: every 4,096-key slice finds the threshold bin b0 from the
//       histogram and keeps its keys whose top bits are >= b0 (all keys
//       above b0 are selected, fewer than k of them; keys in b0 are
//       candidates), written in index order to the slice's list; it also
//       adds key bits 19..8 of its keys in b0 to the row's second-level
//       histogram.
//   sel_final: one workgroup per row reads both histograms, which fix the
//       top 24 bits of the threshold, resolves the last 8 bits over the
//       candidates, then the lowest indices among exact ties, and writes
//       the winners by an ordered compaction of the concatenated slice
//       lists, which are in index order already: no sort is needed.
// Rows whose pool fits the budget skip the radix passes and take the pool.
#include "select_core.h"

namespace hs2 {
namespace {

__global__ __launch_bounds__(256) void sel_init(uint32_t* __restrict__ hist) {
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < kHistRow; i += blockDim.x) hist[(size_t)r * kHistRow + i] = 0u;
}

__global__ __launch_bounds__(256) void sel_hist(const float* __restrict__ scores, int cap,
                                                const int32_t* __restrict__ ctx_len, int tiles,
                                                int n_q, int tile_q, int k_top, int window,
                                                uint32_t* __restrict__ hist) {
  const int r = blockIdx.y;
  const RowGeom g = row_geom(ctx_len, cap, r, tiles, n_q, tile_q, k_top, window);
  const int s0 = blockIdx.x * kSelSlice;
  if (g.kk == 0 || g.kk == g.pe || s0 >= g.pe) return;
  const int s1 = min(g.pe, s0 + kSelSlice);
  __shared__ uint32_t h[kSelBins];
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  const float* row = scores + (size_t)r * cap;
  for (int j = s0 + threadIdx.x; j < s1; j += blockDim.x) atomicAdd(&h[order_key(row[j]) >> 20], 1u);
  __syncthreads();
  uint32_t* gh = hist + (size_t)r * kHistRow;
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x)
    if (h[i] != 0u) atomicAdd(&gh[i], h[i]);
}

template <bool kVec4>
__global__ __launch_bounds__(256) void sel_filter(const float* __restrict__ scores, int cap,
                                                  const int32_t* __restrict__ ctx_len, int tiles,
                                                  int n_q, int tile_q, int k_top, int window,
                                                  uint32_t* __restrict__ hist,
                                                  uint32_t* __restrict__ cnt,
                                                  uint32_t* __restrict__ meta,
                                                  uint2* __restrict__ list, int nslices) {
  const int r = blockIdx.y, s = blockIdx.x;
  const RowGeom g = row_geom(ctx_len, cap, r, tiles, n_q, tile_q, k_top, window);
  if (g.kk == 0 || g.kk == g.pe || s * kSelSlice >= g.pe) return;
  __shared__ FilterLds lds;
  filter_slice<kVec4, false>(scores + (size_t)r * cap, cap, g, s, hist + (size_t)r * kHistRow,
                             cnt + (size_t)r * nslices, meta + 4 * r,
                             list + ((size_t)r * nslices + s) * kSelSlice, lds);
}

__global__ __launch_bounds__(1024) void sel_final(const int32_t* __restrict__ ctx_len, int cap,
                                                  int tiles, int n_q, int tile_q, int k_top,
                                                  int window, const uint32_t* __restrict__ hist,
                                                  const uint32_t* __restrict__ cnt,
                                                  const uint32_t* __restrict__ meta,
                                                  const uint2* __restrict__ list, int nslices,
                                                  int32_t* __restrict__ top_idx,
                                                  int32_t* __restrict__ top_cnt) {
  __shared__ __attribute__((aligned(16))) uint32_t h[256];
  __shared__ uint32_t pre[kMaxSlices + 1];
  __shared__ uint32_t chunk_wins[2 * kStage / 64];
  __shared__ __attribute__((aligned(16))) uint32_t scratch[16];
  __shared__ uint32_t res[6];
  __shared__ uint2 stage[kStage];
  const int r = blockIdx.x;
  const RowGeom g = row_geom(ctx_len, cap, r, tiles, n_q, tile_q, k_top, window);
  const int n = final_select_row<1024>(r, g, k_top, hist, cnt, meta, list, nslices,
                                 top_idx + (size_t)r * k_top, nullptr,
                                 FinalLds{h, pre, chunk_wins, scratch, res, stage});
  if (threadIdx.x == 0) top_cnt[r] = n;
}

}  // namespace

hipError_t launch_select(const hs2_attn_desc& d, const float* scores, const int32_t* ctx_len,
                         int cap, int32_t* top_idx, int32_t* top_cnt, char* ws,
                         uint32_t* hist, bool final_stage, hipStream_t st) {
  const SelectWs w = select_ws(d, cap);
  const int tiles = d.n_q / d.tile_q;
  const int rows = d.batch * tiles;
  const int nslices = select_slices(cap);
  uint32_t* own_hist = reinterpret_cast<uint32_t*>(ws + w.hist_off);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + w.cnt_off);
  uint32_t* meta = reinterpret_cast<uint32_t*>(ws + w.meta_off);
  uint2* list = reinterpret_cast<uint2*>(ws + w.list_off);
  const dim3 grid(nslices, rows);
  if (hist == nullptr) {
    sel_init<<<rows, 256, 0, st>>>(own_hist);
    sel_hist<<<grid, 256, 0, st>>>(scores, cap, ctx_len, tiles, d.n_q, d.tile_q, d.k_top,
                                   d.window, own_hist);
    hist = own_hist;
  }
  if (cap % 4 == 0)
    sel_filter<true><<<grid, 256, 0, st>>>(scores, cap, ctx_len, tiles, d.n_q, d.tile_q, d.k_top,
                                           d.window, hist, cnt, meta, list, nslices);
  else
    sel_filter<false><<<grid, 256, 0, st>>>(scores, cap, ctx_len, tiles, d.n_q, d.tile_q,
                                            d.k_top, d.window, hist, cnt, meta, list, nslices);
  if (final_stage)
    sel_final<<<rows, 1024, 0, st>>>(ctx_len, cap, tiles, d.n_q, d.tile_q, d.k_top, d.window, hist,
                                   cnt, meta, list, nslices, top_idx, top_cnt);
  return hipGetLastError();
}

}  // namespace hs2
