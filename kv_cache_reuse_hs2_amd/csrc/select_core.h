// Row-level selection helpers shared by the selector kernels and the fused
// decode tail: block scans, threshold-bin searches and the final exact
// selection of one row from the filter's candidate lists (see
// select_topk.hip for the method).
#pragma once

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

// find_bin_desc over a histogram held in registers: thread t owns bins
// [kPer t, kPer t + kPer) (threads past the histogram hold zeros).  res must
// not be read between this call and the previous use of the same array
// without a barrier in between.
template <int kPer>
__device__ void find_bin_regs(const uint32_t (&v)[kPer], uint32_t need, uint32_t* scratch,
                              uint32_t* res) {
  const int t = threadIdx.x;
  uint32_t local = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) local += v[e];
  if (t == 0) {
    res[0] = 0u;
    res[1] = 0u;
  }
  const uint32_t suf = block_suffix_sum(local, scratch);
  const uint32_t above = suf - local;
  if (above < need && need <= suf) {
    uint32_t cum = above, bin = 0, cab = 0;
    bool found = false;
#pragma unroll
    for (int e = kPer - 1; e >= 0; --e) {
      if (!found && cum + v[e] >= need) {
        bin = (uint32_t)e;
        cab = cum;
        found = true;
      }
      cum += v[e];
    }
    res[0] = (uint32_t)t * kPer + bin;
    res[1] = cab;
  }
  __syncthreads();
}

constexpr int kMaxSlices = 1024;  // pools up to 4,194,304 keys
constexpr int kStage = 8192;      // list entries held in LDS by the final selection

// LDS of the final selection of one row.
struct FinalLds {
  uint32_t* h;           // [2048], 16-byte aligned: bits 7..0, then the tie passes
  uint32_t* pre;         // [kMaxSlices + 1] slice offsets
  uint32_t* chunk_wins;  // [kStage / 64]
  uint32_t* scratch;     // [16], 16-byte aligned
  uint32_t* res;         // [6]: three result pairs
  uint2* stage;          // [kStage] the candidate list
};

// Final exact selection of row r by a workgroup of kThreads threads: the
// winners go to out[0 .. n) in ascending index order, -1 after them up to
// k_top (when out is given), and to win[0 .. n) (when win, in LDS, is given).
// Returns n to every thread.
template <int kThreads>
__device__ int final_select_row(int r, const RowGeom& g, int k_top,
                                const uint32_t* __restrict__ hist,
                                const uint32_t* __restrict__ cnt,
                                const uint32_t* __restrict__ meta,
                                const uint2* __restrict__ list, int nslices,
                                int32_t* __restrict__ out, int32_t* win, const FinalLds& L) {
  static_assert(kThreads % 64 == 0 && kSelBins % (4 * kThreads) == 0, "whole waves, 4k bins each");
  constexpr int kWaves = kThreads / 64;
  constexpr int kBinsPer = kSelBins / kThreads;
  const int t = threadIdx.x;
  if (g.kk == 0 || g.kk == g.pe) {
    for (int i = t; i < k_top; i += blockDim.x) {
      if (out != nullptr) out[i] = i < g.kk ? i : -1;
      if (win != nullptr && i < g.kk) win[i] = i;
    }
    if (win != nullptr) __syncthreads();
    return g.kk;
  }
  uint32_t* h = L.h;
  uint32_t* pre = L.pre;
  uint32_t* chunk_wins = L.chunk_wins;
  uint32_t* scratch = L.scratch;
  uint32_t* res_b = L.res;
  uint32_t* res_c = L.res + 2;
  uint32_t* res = L.res + 4;
  uint2* stage = L.stage;
  const int lane = t & 63, wave = t >> 6;
  const int ns = (g.pe + kSelSlice - 1) / kSelSlice;
  const uint2* lr = list + (size_t)r * nslices * kSelSlice;

  // Everything that does not depend on another load is fetched at once: the
  // threshold bin b0 that sel_filter found, the second-level histogram (bins
  // kBinsPer t .. kBinsPer t + kBinsPer - 1 per thread), the slice counts,
  // and the head of each slice list this wave will copy first (slices
  // wave + kWaves u for u < kHeads, entries 0..63).
  const uint32_t* hrow = hist + (size_t)r * kHistRow;
  uint32_t v2[kBinsPer];
#pragma unroll
  for (int i = 0; i < kBinsPer; i += 4) {
    const u32x4 x2 = *reinterpret_cast<const u32x4*>(hrow + kSelBins + kBinsPer * t + i);
    v2[i] = x2.x;
    v2[i + 1] = x2.y;
    v2[i + 2] = x2.z;
    v2[i + 3] = x2.w;
  }
  const uint32_t b0 = meta[4 * r], above0 = meta[4 * r + 1];
  constexpr int kHeads = 8;
  uint2 head[kHeads];
#pragma unroll
  for (int u = 0; u < kHeads; ++u) {
    const int sl = wave + kWaves * u;
    if (sl < ns) head[u] = lr[(size_t)sl * kSelSlice + lane];
  }
  for (int i = t; i < 256; i += kThreads) h[i] = 0u;  // key bits 7..0, counted while staging

  // Slice offsets: one wave scans the counts 64 at a time.
  if (wave == 0) {
    uint32_t carry = 0;
    for (int c0 = 0; c0 < ns; c0 += 64) {
      const uint32_t c = (c0 + lane < ns) ? cnt[(size_t)r * nslices + c0 + lane] : 0u;
      uint32_t incl = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (c0 + lane < ns) pre[c0 + lane] = carry + incl - c;
      carry += __shfl(incl, 63);
    }
    if (lane == 0) pre[ns] = carry;
  }

  // Bits 19..8 of the threshold among the keys of b0.
  const uint32_t need0 = (uint32_t)g.kk - above0;
  find_bin_regs(v2, need0, scratch, res_b);  // its barriers also publish pre[]
  const uint32_t b1 = res_b[0];
  const uint32_t need1 = need0 - res_b[1];
  const uint32_t top24 = (b0 << 12) | b1;
  const uint32_t total = pre[ns];

  auto entry_global = [&](uint32_t gi) -> uint2 {
    int lo = 0, hi = ns - 1;  // last slice with pre[s] <= gi
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= gi) lo = mid;
      else hi = mid - 1;
    }
    return lr[(size_t)lo * kSelSlice + (gi - pre[lo])];
  };
  // The list is read twice more: keep it in LDS when it fits (the usual
  // case: keys above the threshold bin plus that bin).  Each wave copies
  // whole slices, kHeads at a time so that their loads overlap (the first
  // kHeads from the heads loaded above), and counts key bits 7..0 of the
  // candidates that match the top 24 bits on the way.
  const bool staged = total <= (uint32_t)kStage;
  auto put = [&](uint32_t pos, uint2 e) {
    stage[pos] = e;
    if ((e.x >> 8) == top24) atomicAdd(&h[e.x & 0xFFu], 1u);
  };
  if (staged) {
    for (int sl0 = wave; sl0 < ns; sl0 += kHeads * kWaves) {
      uint2 e[kHeads];
      uint32_t n[kHeads];
#pragma unroll
      for (int u = 0; u < kHeads; ++u) {
        const int sl = sl0 + kWaves * u;
        n[u] = sl < ns ? pre[sl + 1] - pre[sl] : 0u;
        if (sl0 == wave) e[u] = head[u];
        else if ((uint32_t)lane < n[u]) e[u] = lr[(size_t)sl * kSelSlice + lane];
      }
#pragma unroll
      for (int u = 0; u < kHeads; ++u) {
        const int sl = sl0 + kWaves * u;
        if ((uint32_t)lane < n[u]) put(pre[sl] + lane, e[u]);
        for (uint32_t i = 64 + lane; i < n[u]; i += 64) put(pre[sl] + i, lr[(size_t)sl * kSelSlice + i]);
      }
    }
  } else {
    for (uint32_t i = t; i < total; i += blockDim.x) {
      const uint32_t kx = entry_global(i).x;
      if ((kx >> 8) == top24) atomicAdd(&h[kx & 0xFFu], 1u);
    }
  }
  __syncthreads();
  auto entry = [&](uint32_t gi) -> uint2 { return staged ? stage[gi] : entry_global(gi); };

  // Key bits 7..0 among the candidates that match the top 24 bits.
  uint32_t v3[4] = {0u, 0u, 0u, 0u};
  if (t < 64) {
    const u32x4 x3 = *reinterpret_cast<const u32x4*>(&h[4 * t]);
    v3[0] = x3.x;
    v3[1] = x3.y;
    v3[2] = x3.z;
    v3[3] = x3.w;
  }
  find_bin_regs(v3, need1, scratch, res_c);
  const uint32_t b2 = res_c[0];
  const uint32_t need2 = need1 - res_c[1];
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

  // Ordered compaction of the winners.  A staged list is cut into 64-entry
  // chunks, one lane per entry: a ballot counts each chunk's winners, and a
  // winner's place is the winners of earlier chunks plus those of lower
  // lanes.  A list left in global memory goes through one block prefix sum
  // over runs of consecutive entries.
  auto wins = [&](uint2 c) { return c.x > tau || (c.x == tau && c.y <= idx_thr); };
  uint32_t base;
  if (staged) {
    const int nchunks = (int)((total + 63) / 64);
    uint64_t mask[kStage / 64 / kWaves];
#pragma unroll
    for (int u = 0; u < kStage / 64 / kWaves; ++u) {
      const int ch = wave + kWaves * u;
      const uint32_t e = 64u * ch + lane;
      const bool w = ch < nchunks && e < total && wins(stage[e]);
      mask[u] = __ballot(w);
      if (ch < nchunks && lane == 0) chunk_wins[ch] = (uint32_t)__popcll(mask[u]);
    }
    __syncthreads();
    // Winners of the chunks before each chunk: one wave scans the counts in
    // place (res[0] gets the total; the earlier results there are consumed).
    if (wave == 0) {
      uint32_t carry = 0;
      for (int c0 = 0; c0 < nchunks; c0 += 64) {
        const uint32_t c = (c0 + lane < nchunks) ? chunk_wins[c0 + lane] : 0u;
        uint32_t incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t o = __shfl_up(incl, off);
          if (lane >= off) incl += o;
        }
        if (c0 + lane < nchunks) chunk_wins[c0 + lane] = carry + incl - c;
        carry += __shfl(incl, 63);
      }
      if (lane == 0) res_b[0] = carry;
    }
    __syncthreads();
    base = res_b[0];
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int u = 0; u < kStage / 64 / kWaves; ++u) {
      const int ch = wave + kWaves * u;
      if (ch >= nchunks) break;
      const uint32_t before = chunk_wins[ch];
      if ((mask[u] >> lane) & 1ull) {
        const uint32_t pos = before + (uint32_t)__popcll(mask[u] & lower);
        if (pos < (uint32_t)k_top) {
          if (out != nullptr) out[pos] = (int32_t)stage[64u * ch + lane].y;
          if (win != nullptr) win[pos] = (int32_t)stage[64u * ch + lane].y;
        }
      }
    }
  } else {
    const uint32_t per = (total + blockDim.x - 1) / blockDim.x;
    const uint32_t e0 = min(total, t * per), e1 = min(total, e0 + per);
    uint32_t mine = 0;
    for (uint32_t e = e0; e < e1; ++e) mine += wins(entry(e)) ? 1u : 0u;
    uint32_t pos = block_prefix_sum(mine, scratch, &base);
    for (uint32_t e = e0; e < e1; ++e) {
      const uint2 c = entry(e);
      if (wins(c)) {
        if (pos < (uint32_t)k_top) {
          if (out != nullptr) out[pos] = (int32_t)c.y;
          if (win != nullptr) win[pos] = (int32_t)c.y;
        }
        ++pos;
      }
    }
  }
  if (out != nullptr)
    for (int i = (int)min(base, (uint32_t)k_top) + t; i < k_top; i += blockDim.x) out[i] = -1;
  if (win != nullptr) __syncthreads();
  return (int)min(base, (uint32_t)k_top);
}

}  // namespace
}  // namespace hs2
