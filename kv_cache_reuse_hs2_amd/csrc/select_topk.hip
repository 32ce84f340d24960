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
//       candidates), written in index order to the slice's list.
//   sel_final: one workgroup per row resolves the remaining 20 key bits over
//       the candidates, then the lowest indices among exact ties, and writes
//       the winners by an ordered compaction of the concatenated slice
//       lists, which are in index order already: no sort is needed.
// Rows whose pool fits the budget skip the radix passes and take the pool.
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

// Inclusive suffix sum of v over the block (all threads call; scratch holds
// one word per wave).  Returns the sum over threads >= t.
__device__ __forceinline__ uint32_t block_suffix_sum(uint32_t v, uint32_t* scratch) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, nw = blockDim.x >> 6;
  uint32_t s = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_down(s, off);
    if (lane + off < 64) s += o;
  }
  if (lane == 0) scratch[wave] = s;
  __syncthreads();
  uint32_t later = 0;
  for (int w = wave + 1; w < nw; ++w) later += scratch[w];
  __syncthreads();
  return s + later;
}

// Exclusive prefix sum of v over the block; *total gets the block sum.
__device__ __forceinline__ uint32_t block_prefix_sum(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, nw = blockDim.x >> 6;
  uint32_t s = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(s, off);
    if (lane >= off) s += o;
  }
  if (lane == 63) scratch[wave] = s;
  __syncthreads();
  uint32_t before = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    if (w < wave) before += scratch[w];
    all += scratch[w];
  }
  __syncthreads();
  *total = all;
  return s - v + before;
}

// Search, from the highest bin down, for the bin where the running count
// reaches `need` (1 <= need <= total).  Threads [0, nt) own nbins/nt
// consecutive bins.  res = {bin, count strictly above it}.  All threads call.
__device__ void find_bin_desc(const uint32_t* hist, int nbins, uint32_t need, uint32_t* scratch,
                              uint32_t* res) {
  const int t = threadIdx.x;
  const int nt = min((int)blockDim.x, nbins);
  const int per = nbins / nt;
  uint32_t local = 0;
  if (t < nt)
    for (int i = 0; i < per; ++i) local += hist[t * per + i];
  if (t == 0) {
    res[0] = 0u;
    res[1] = 0u;
  }
  const uint32_t suf = block_suffix_sum(local, scratch);
  if (t < nt) {
    const uint32_t above = suf - local;
    if (above < need && need <= suf) {
      uint32_t cum = above;
      for (int i = per - 1; i >= 0; --i) {
        const uint32_t c = hist[t * per + i];
        if (cum + c >= need) {
          res[0] = t * per + i;
          res[1] = cum;
          break;
        }
        cum += c;
      }
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void sel_init(uint32_t* __restrict__ hist) {
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) hist[(size_t)r * kSelBins + i] = 0u;
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

constexpr int kPer = kSelSlice / 256;  // keys per thread in sel_filter

template <bool kVec4>
__global__ __launch_bounds__(256) void sel_filter(const float* __restrict__ scores, int cap,
                                                  const int32_t* __restrict__ ctx_len, int tiles,
                                                  int n_q, int tile_q, int k_top, int window,
                                                  const uint32_t* __restrict__ hist,
                                                  uint32_t* __restrict__ cnt,
                                                  uint2* __restrict__ list, int nslices) {
  const int r = blockIdx.y, s = blockIdx.x;
  const RowGeom g = row_geom(ctx_len, cap, r, tiles, n_q, tile_q, k_top, window);
  const int s0 = s * kSelSlice;
  if (g.kk == 0 || g.kk == g.pe || s0 >= g.pe) return;
  __shared__ uint32_t scratch[8];
  __shared__ uint32_t res[2];
  find_bin_desc(hist + (size_t)r * kSelBins, kSelBins, (uint32_t)g.kk, scratch, res);
  const uint32_t b0 = res[0];
  // Thread t owns the 16 consecutive keys s0 + 16t .. s0 + 16t + 15.
  const int j0 = s0 + kPer * threadIdx.x;
  const float* row = scores + (size_t)r * cap;
  uint32_t key[kPer];
  if (kVec4 && j0 + kPer <= g.pe) {
#pragma unroll
    for (int e = 0; e < kPer; e += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + j0 + e);
      key[e] = order_key(v.x);
      key[e + 1] = order_key(v.y);
      key[e + 2] = order_key(v.z);
      key[e + 3] = order_key(v.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPer; ++e) key[e] = (j0 + e < g.pe) ? order_key(row[j0 + e]) : 0u;
  }
  uint32_t keep = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) keep += (j0 + e < g.pe && (key[e] >> 20) >= b0) ? 1u : 0u;
  uint32_t total;
  uint32_t pos = block_prefix_sum(keep, scratch, &total);
  uint2* out = list + ((size_t)r * nslices + s) * kSelSlice;
#pragma unroll
  for (int e = 0; e < kPer; ++e)
    if (j0 + e < g.pe && (key[e] >> 20) >= b0) out[pos++] = make_uint2(key[e], (uint32_t)(j0 + e));
  if (threadIdx.x == 0) cnt[(size_t)r * nslices + s] = total;
}

constexpr int kMaxSlices = 1024;  // pools up to 4,194,304 keys
constexpr int kStage = 8192;      // list entries held in LDS by sel_final

__global__ __launch_bounds__(1024) void sel_final(const int32_t* __restrict__ ctx_len, int cap,
                                                  int tiles, int n_q, int tile_q, int k_top,
                                                  int window, const uint32_t* __restrict__ hist,
                                                  const uint32_t* __restrict__ cnt,
                                                  const uint2* __restrict__ list, int nslices,
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
  __shared__ uint32_t pre[kMaxSlices + 1];
  __shared__ uint32_t scratch[16];
  __shared__ uint32_t res[2];

  // Offsets of the slice lists; their concatenation is in index order.
  const int ns = (g.pe + kSelSlice - 1) / kSelSlice;
  uint32_t total = 0;
  {
    const uint32_t c = (t < ns) ? cnt[(size_t)r * nslices + t] : 0u;
    const uint32_t p = block_prefix_sum(c, scratch, &total);
    if (t < ns) pre[t] = p;
    if (t == 0) pre[ns] = total;
    __syncthreads();
  }
  const uint2* lr = list + (size_t)r * nslices * kSelSlice;
  auto entry_global = [&](uint32_t gi) -> uint2 {
    int lo = 0, hi = ns - 1;  // last slice with pre[s] <= gi
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= gi) lo = mid;
      else hi = mid - 1;
    }
    return lr[(size_t)lo * kSelSlice + (gi - pre[lo])];
  };
  // The radix passes below read the list several times: keep it in LDS when
  // it fits (the usual case: keys above the threshold bin plus that bin).
  __shared__ uint2 stage[kStage];
  const bool staged = total <= (uint32_t)kStage;
  if (staged) {
    for (uint32_t e = t; e < total; e += blockDim.x) stage[e] = entry_global(e);
    __syncthreads();
  }
  auto entry = [&](uint32_t gi) -> uint2 { return staged ? stage[gi] : entry_global(gi); };

  // Threshold bin b0 and the count above it, as in sel_filter.
  for (int i = t; i < kSelBins; i += blockDim.x) h[i] = hist[(size_t)r * kSelBins + i];
  __syncthreads();
  find_bin_desc(h, kSelBins, (uint32_t)g.kk, scratch, res);
  const uint32_t b0 = res[0];
  const uint32_t need0 = (uint32_t)g.kk - res[1];

  // Key bits 19..8 among the candidates (top bits == b0).
  for (int i = t; i < kSelBins; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  for (uint32_t e = t; e < total; e += blockDim.x) {
    const uint32_t kx = entry(e).x;
    if ((kx >> 20) == b0) atomicAdd(&h[(kx >> 8) & 0xFFFu], 1u);
  }
  __syncthreads();
  find_bin_desc(h, kSelBins, need0, scratch, res);
  const uint32_t b1 = res[0];
  const uint32_t need1 = need0 - res[1];
  const uint32_t top24 = (b0 << 12) | b1;
  // Key bits 7..0 among the candidates that match the top 24 bits.
  for (int i = t; i < 256; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  for (uint32_t e = t; e < total; e += blockDim.x) {
    const uint32_t kx = entry(e).x;
    if ((kx >> 8) == top24) atomicAdd(&h[kx & 0xFFu], 1u);
  }
  __syncthreads();
  find_bin_desc(h, 256, need1, scratch, res);
  const uint32_t b2 = res[0];
  const uint32_t need2 = need1 - res[1];
  const uint32_t ties = h[b2];
  const uint32_t tau = (top24 << 8) | b2;
  __syncthreads();

  // Among keys equal to tau keep the need2 lowest indices: radix-select the
  // need2-th smallest index (digits of 11/10/10 bits, searched from the top
  // on the reversed digit).
  uint32_t idx_thr = 0xFFFFFFFFu;
  if (need2 < ties) {
    uint32_t prefix = 0, need = need2;
    for (int p = 0; p < 3; ++p) {
      const int sh = (p == 0) ? 20 : (p == 1 ? 10 : 0);
      const uint32_t nb = (p == 0) ? 2048u : 1024u;
      for (int i = t; i < (int)nb; i += blockDim.x) h[i] = 0u;
      __syncthreads();
      for (uint32_t e = t; e < total; e += blockDim.x) {
        const uint2 c = entry(e);
        if (c.x != tau) continue;
        // Index bits above this digit must match the digits already fixed.
        if (p > 0 && (c.y >> (sh + 10)) != prefix) continue;
        atomicAdd(&h[nb - 1u - ((c.y >> sh) & (nb - 1u))], 1u);
      }
      __syncthreads();
      find_bin_desc(h, nb, need, scratch, res);
      const uint32_t dgt = nb - 1u - res[0];
      need -= res[1];
      prefix = (p == 0) ? dgt : ((prefix << 10) | dgt);
      __syncthreads();
    }
    idx_thr = prefix;
  }

  // Ordered compaction of the winners.
  uint32_t base = 0;
  for (uint32_t r0 = 0; r0 < total; r0 += blockDim.x) {
    const uint32_t e = r0 + t;
    bool win = false;
    uint32_t idx = 0;
    if (e < total) {
      const uint2 c = entry(e);
      win = c.x > tau || (c.x == tau && c.y <= idx_thr);
      idx = c.y;
    }
    uint32_t round_total;
    const uint32_t pos = base + block_prefix_sum(win ? 1u : 0u, scratch, &round_total);
    if (win && pos < (uint32_t)k_top) out[pos] = (int32_t)idx;
    base += round_total;
  }
  for (int i = (int)min(base, (uint32_t)k_top) + t; i < k_top; i += blockDim.x) out[i] = -1;
  if (t == 0) top_cnt[r] = (int32_t)min(base, (uint32_t)k_top);
}

}  // namespace

hipError_t launch_select(const hs2_attn_desc& d, const float* scores, const int32_t* ctx_len,
                         int cap, int32_t* top_idx, int32_t* top_cnt, char* ws,
                         const uint32_t* hist, hipStream_t st) {
  const SelectWs w = select_ws(d, cap);
  const int tiles = d.n_q / d.tile_q;
  const int rows = d.batch * tiles;
  const int nslices = select_slices(cap);
  uint32_t* own_hist = reinterpret_cast<uint32_t*>(ws + w.hist_off);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + w.cnt_off);
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
                                           d.window, hist, cnt, list, nslices);
  else
    sel_filter<false><<<grid, 256, 0, st>>>(scores, cap, ctx_len, tiles, d.n_q, d.tile_q,
                                            d.k_top, d.window, hist, cnt, list, nslices);
  sel_final<<<rows, 1024, 0, st>>>(ctx_len, cap, tiles, d.n_q, d.tile_q, d.k_top, d.window, hist,
                                   cnt, list, nslices, top_idx, top_cnt);
  return hipGetLastError();
}

}  // namespace hs2
