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
//   1. sel_hist:   per-row histogram of the top 12 bits (LDS per workgroup,
//                  merged with integer atomics: order-independent result).
//   2. sel_filter: every workgroup finds the threshold bin b0 from that
//                  histogram and splits its slice into keys above b0 (always
//                  selected, fewer than k) and candidates inside b0.
//   3. sel_final:  one workgroup per row resolves the remaining 20 key bits
//                  over the candidates, then the lowest indices among exact
//                  ties, gathers the k winners and bitonic-sorts them into
//                  ascending index order.
// Rows whose pool fits the budget skip 1-2 and take the whole pool.
#include "hs2_internal.h"

namespace hs2 {
namespace {

struct RowGeom {
  int pe;  // pool end (exclusive)
  int kk;  // keys to select = min(k_top, pe)
};

__device__ __forceinline__ RowGeom row_geom(const int32_t* ctx_len, int cap, int r, int tiles,
                                            int n_q, int tile_q, int k_top, int window) {
  const int b = r / tiles, g = r % tiles;
  const int N = clamp_ctx(ctx_len, b, cap);
  const int p0 = N - n_q + g * tile_q;
  int pe = p0 - window + 1;
  if (pe < 0) pe = 0;
  RowGeom w;
  w.pe = pe;
  w.kk = min(k_top, pe);
  return w;
}

// Block-wide search, from the highest bin down, for the bin where the running
// count reaches `need`.  Returns (bin, count strictly above it) through LDS.
// Threads [0, nt) each own nbins/nt consecutive bins; all threads must call.
__device__ void find_bin_desc(const uint32_t* hist, int nbins, uint32_t need, uint32_t* scan,
                              uint32_t* result) {
  const int t = threadIdx.x;
  const int nt = min((int)blockDim.x, nbins);
  const int per = nbins / nt;
  uint32_t local = 0;
  if (t < nt)
    for (int i = 0; i < per; ++i) local += hist[t * per + i];
  if (t == 0) {
    result[0] = 0;
    result[1] = 0;
  }
  scan[t] = (t < nt) ? local : 0u;
  __syncthreads();
  // Inclusive suffix sum over scan[0..blockDim) (Hillis-Steele).
  for (int off = 1; off < (int)blockDim.x; off <<= 1) {
    const uint32_t add = (t + off < (int)blockDim.x) ? scan[t + off] : 0u;
    __syncthreads();
    scan[t] += add;
    __syncthreads();
  }
  if (t < nt) {
    const uint32_t above = scan[t] - local;  // count in bins owned by threads > t
    if (above < need && need <= above + local) {
      uint32_t cum = above;
      for (int i = per - 1; i >= 0; --i) {
        const uint32_t c = hist[t * per + i];
        if (cum + c >= need) {
          result[0] = t * per + i;
          result[1] = cum;
          break;
        }
        cum += c;
      }
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void sel_init(uint32_t* __restrict__ hist,
                                                uint32_t* __restrict__ ctr, int rows) {
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) hist[(size_t)r * kSelBins + i] = 0u;
  if (threadIdx.x < 4) ctr[r * 4 + threadIdx.x] = 0u;
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
  uint32_t* gh = hist + (size_t)r * kSelBins;
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x)
    if (h[i] != 0u) atomicAdd(&gh[i], h[i]);
}

constexpr int kFilterPer = kSelSlice / 256;

__global__ __launch_bounds__(256) void sel_filter(const float* __restrict__ scores, int cap,
                                                  const int32_t* __restrict__ ctx_len, int tiles,
                                                  int n_q, int tile_q, int k_top, int window,
                                                  const uint32_t* __restrict__ hist,
                                                  uint32_t* __restrict__ ctr,
                                                  int32_t* __restrict__ greater,
                                                  uint2* __restrict__ cand) {
  const int r = blockIdx.y;
  const RowGeom g = row_geom(ctx_len, cap, r, tiles, n_q, tile_q, k_top, window);
  const int s0 = blockIdx.x * kSelSlice;
  if (g.kk == 0 || g.kk == g.pe || s0 >= g.pe) return;
  const int s1 = min(g.pe, s0 + kSelSlice);
  __shared__ uint32_t scan[256];
  __shared__ uint32_t res[2];
  __shared__ uint32_t lcnt[2], base[2];
  find_bin_desc(hist + (size_t)r * kSelBins, kSelBins, (uint32_t)g.kk, scan, res);
  const uint32_t b0 = res[0];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ctr[r * 4 + 2] = b0;
    ctr[r * 4 + 3] = res[1];
  }
  if (threadIdx.x < 2) lcnt[threadIdx.x] = 0u;
  __syncthreads();
  const float* row = scores + (size_t)r * cap;
  uint32_t key[kFilterPer];
  int slot[kFilterPer];
#pragma unroll
  for (int e = 0; e < kFilterPer; ++e) {
    const int j = s0 + e * 256 + threadIdx.x;
    slot[e] = -1;
    key[e] = 0u;
    if (j < s1) {
      key[e] = order_key(row[j]);
      const uint32_t d = key[e] >> 20;
      if (d > b0) slot[e] = (int)atomicAdd(&lcnt[0], 1u);
      else if (d == b0) slot[e] = (int)atomicAdd(&lcnt[1], 1u);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    base[0] = lcnt[0] ? atomicAdd(&ctr[r * 4 + 0], lcnt[0]) : 0u;
    base[1] = lcnt[1] ? atomicAdd(&ctr[r * 4 + 1], lcnt[1]) : 0u;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kFilterPer; ++e) {
    if (slot[e] < 0) continue;
    const int j = s0 + e * 256 + threadIdx.x;
    if ((key[e] >> 20) > b0) {
      const uint32_t p = base[0] + slot[e];
      if (p < (uint32_t)kMaxTop) greater[(size_t)r * kMaxTop + p] = j;
    } else {
      cand[(size_t)r * cap + base[1] + slot[e]] = make_uint2(key[e], (uint32_t)j);
    }
  }
}

__global__ __launch_bounds__(1024) void sel_final(const int32_t* __restrict__ ctx_len, int cap,
                                                  int tiles, int n_q, int tile_q, int k_top,
                                                  int window, const uint32_t* __restrict__ ctr,
                                                  const int32_t* __restrict__ greater,
                                                  const uint2* __restrict__ cand,
                                                  int32_t* __restrict__ top_idx,
                                                  int32_t* __restrict__ top_cnt) {
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const RowGeom g = row_geom(ctx_len, cap, r, tiles, n_q, tile_q, k_top, window);
  int32_t* out = top_idx + (size_t)r * k_top;
  if (g.kk == 0 || g.kk == g.pe) {
    for (int i = t; i < k_top; i += blockDim.x) out[i] = i < g.kk ? i : -1;
    if (t == 0) top_cnt[r] = g.kk;
    return;
  }
  __shared__ uint32_t h[kSelBins];
  __shared__ uint32_t scan[1024];
  __shared__ uint32_t res[2];
  __shared__ int32_t sel[kMaxTop];
  __shared__ uint32_t nsel;

  const uint32_t b0 = ctr[r * 4 + 2];
  const uint32_t g0 = ctr[r * 4 + 3];
  const uint32_t c0 = ctr[r * 4 + 1];
  const uint2* cr = cand + (size_t)r * cap;
  const uint32_t need0 = (uint32_t)g.kk - g0;

  // Key bits 19..8 among the candidates (all of which share bits 31..20 = b0).
  for (int i = t; i < kSelBins; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  for (uint32_t e = t; e < c0; e += blockDim.x) atomicAdd(&h[(cr[e].x >> 8) & 0xFFFu], 1u);
  __syncthreads();
  find_bin_desc(h, kSelBins, need0, scan, res);
  const uint32_t b1 = res[0];
  const uint32_t need1 = need0 - res[1];
  // Key bits 7..0 among the candidates that match b1.
  for (int i = t; i < 256; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  for (uint32_t e = t; e < c0; e += blockDim.x) {
    const uint32_t kx = cr[e].x;
    if (((kx >> 8) & 0xFFFu) == b1) atomicAdd(&h[kx & 0xFFu], 1u);
  }
  __syncthreads();
  find_bin_desc(h, 256, need1, scan, res);
  const uint32_t b2 = res[0];
  const uint32_t need2 = need1 - res[1];
  const uint32_t ties = h[b2];
  const uint32_t tau = (b0 << 20) | (b1 << 8) | b2;
  __syncthreads();

  // Among keys equal to tau keep the need2 lowest indices: radix-select the
  // need2-th smallest index (digits 11/10/10 bits, searched from the top on
  // the reversed digit).
  uint32_t idx_thr = 0xFFFFFFFFu;
  if (need2 < ties) {
    uint32_t prefix = 0, need = need2;
    const int shifts[3] = {20, 10, 0};
    const uint32_t widths[3] = {2048u, 1024u, 1024u};
    for (int p = 0; p < 3; ++p) {
      const int sh = shifts[p];
      const uint32_t nb = widths[p];
      for (int i = t; i < (int)nb; i += blockDim.x) h[i] = 0u;
      __syncthreads();
      for (uint32_t e = t; e < c0; e += blockDim.x) {
        const uint2 c = cr[e];
        if (c.x != tau) continue;
        // Index bits above this digit must match the digits already fixed.
        if (p > 0 && (c.y >> (sh + 10)) != prefix) continue;
        const uint32_t dgt = (c.y >> sh) & (nb - 1u);
        atomicAdd(&h[nb - 1u - dgt], 1u);
      }
      __syncthreads();
      find_bin_desc(h, nb, need, scan, res);
      const uint32_t dgt = nb - 1u - res[0];
      need -= res[1];
      prefix = (p == 0) ? dgt : ((prefix << 10) | dgt);
      __syncthreads();
    }
    idx_thr = prefix;
  }

  // Gather the winners: keys above b0, then candidates above tau or tied
  // with an index not beyond idx_thr.
  if (t == 0) nsel = 0u;
  __syncthreads();
  for (uint32_t e = t; e < g0 && e < (uint32_t)kMaxTop; e += blockDim.x) {
    const uint32_t p = atomicAdd(&nsel, 1u);
    if (p < (uint32_t)kMaxTop) sel[p] = greater[(size_t)r * kMaxTop + e];
  }
  for (uint32_t e = t; e < c0; e += blockDim.x) {
    const uint2 c = cr[e];
    if (c.x > tau || (c.x == tau && c.y <= idx_thr)) {
      const uint32_t p = atomicAdd(&nsel, 1u);
      if (p < (uint32_t)kMaxTop) sel[p] = (int32_t)c.y;
    }
  }
  __syncthreads();
  const int kk = g.kk;
  int n2 = 1;
  while (n2 < kk) n2 <<= 1;
  for (int i = kk + t; i < n2; i += blockDim.x) sel[i] = 0x7FFFFFFF;
  __syncthreads();
  // Bitonic sort of sel[0..n2) ascending.
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < (n2 >> 1); i += blockDim.x) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool asc = (lo & size) == 0;
        const int32_t a = sel[lo], bv = sel[hi];
        if ((a > bv) == asc) {
          sel[lo] = bv;
          sel[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = t; i < k_top; i += blockDim.x) out[i] = i < kk ? sel[i] : -1;
  if (t == 0) top_cnt[r] = kk;
}

}  // namespace

hipError_t launch_select(const hs2_attn_desc& d, const float* scores, const int32_t* ctx_len,
                         int cap, int32_t* top_idx, int32_t* top_cnt, char* ws, hipStream_t st) {
  const SelectWs w = select_ws(d, cap);
  const int tiles = d.n_q / d.tile_q;
  const int rows = d.batch * tiles;
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + w.hist_off);
  uint32_t* ctr = reinterpret_cast<uint32_t*>(ws + w.ctr_off);
  int32_t* greater = reinterpret_cast<int32_t*>(ws + w.greater_off);
  uint2* cand = reinterpret_cast<uint2*>(ws + w.cand_off);
  const int nslices = (cap + kSelSlice - 1) / kSelSlice;
  const dim3 grid(nslices, rows);
  sel_init<<<rows, 256, 0, st>>>(hist, ctr, rows);
  sel_hist<<<grid, 256, 0, st>>>(scores, cap, ctx_len, tiles, d.n_q, d.tile_q, d.k_top, d.window,
                                 hist);
  sel_filter<<<grid, 256, 0, st>>>(scores, cap, ctx_len, tiles, d.n_q, d.tile_q, d.k_top,
                                   d.window, hist, ctr, greater, cand);
  sel_final<<<rows, 1024, 0, st>>>(ctx_len, cap, tiles, d.n_q, d.tile_q, d.k_top, d.window, ctr,
                                   greater, cand, top_idx, top_cnt);
  return hipGetLastError();
}

}  // namespace hs2
