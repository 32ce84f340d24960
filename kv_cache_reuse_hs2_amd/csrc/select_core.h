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

// The candidate filter of one 4,096-key slice s of a row (256 threads): it
// finds the threshold bin b0 (top 12 key bits) from the row's first-level
// histogram, writes the slice's keys whose top bits are >= b0, in index
// order, as (key, index) pairs to list_s and their count to cnt_r[s]
// (slice 0 also writes b0 and the pool count above b0 to meta_r), and adds
// key bits 19..8 of its keys in b0 to the row's second-level histogram.
// kCoherent: the scores and the histogram were written by other workgroups
// of the same launch, so they are read at device scope (sc1); kVec4: the row
// is 16-byte aligned (the row length is a multiple of 4).
constexpr int kFiltPer = kSelSlice / 256;  // keys per thread
// Above this many threshold-bin keys in a slice, the second-level histogram
// is merged in LDS first instead of one global atomic per key.
constexpr uint32_t kDirectHist2 = 256;

struct FilterLds {
  uint32_t scratch[8];
  uint32_t res[2];
  uint32_t h2[kSelBins];
};

template <bool kVec4, bool kCoherent>
__device__ void filter_slice(const float* __restrict__ row, int cap, const RowGeom& g, int s,
                             uint32_t* __restrict__ hrow, uint32_t* __restrict__ cnt_r,
                             uint32_t* __restrict__ meta_r, uint2* __restrict__ list_s,
                             FilterLds& L) {
  static_assert(kSelBins == 16 * 256 && kFiltPer == 16, "sixteen keys and bins per thread");
  const int s0 = s * kSelSlice;
  // Thread t owns the 16 consecutive keys s0 + 16t .. s0 + 16t + 15; they are
  // loaded first so that the loads overlap the threshold search.
  const int j0 = s0 + kFiltPer * threadIdx.x;
  uint32_t key[kFiltPer];
  uint32_t hv[16];
  if constexpr (kCoherent) {
    // The row's cap scores (keys past the pool end are loaded, never kept).
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(row, (uint32_t)cap * 4u);
    const __amdgpu_buffer_rsrc_t rh = buffer_rsrc(hrow, kSelBins * 4u);
    if (kVec4) {
#pragma unroll
      for (int e = 0; e < kFiltPer; e += 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, (j0 + e) * 4, 0, kSc1);
#pragma unroll
        for (int u = 0; u < 4; ++u) key[e + u] = order_key(__uint_as_float(v[u]));
      }
    } else {
#pragma unroll
      for (int e = 0; e < kFiltPer; ++e)
        key[e] = order_key(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (j0 + e) * 4, 0, kSc1)));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rh, (16 * threadIdx.x + 4 * i) * 4, 0, kSc1);
#pragma unroll
      for (int u = 0; u < 4; ++u) hv[4 * i + u] = x[u];
    }
  } else {
    if (kVec4 && j0 + kFiltPer <= g.pe) {
#pragma unroll
      for (int e = 0; e < kFiltPer; e += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(row + j0 + e);
        key[e] = order_key(v.x);
        key[e + 1] = order_key(v.y);
        key[e + 2] = order_key(v.z);
        key[e + 3] = order_key(v.w);
      }
    } else {
#pragma unroll
      for (int e = 0; e < kFiltPer; ++e) key[e] = (j0 + e < g.pe) ? order_key(row[j0 + e]) : 0u;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(hrow + 16 * threadIdx.x + 4 * i);
      hv[4 * i] = x.x;
      hv[4 * i + 1] = x.y;
      hv[4 * i + 2] = x.z;
      hv[4 * i + 3] = x.w;
    }
  }
  find_bin_regs(hv, (uint32_t)g.kk, L.scratch, L.res);
  const uint32_t b0 = L.res[0];
  uint32_t keep = 0, in_b0 = 0;
#pragma unroll
  for (int e = 0; e < kFiltPer; ++e) {
    const bool valid = j0 + e < g.pe;
    keep += (valid && (key[e] >> 20) >= b0) ? 1u : 0u;
    in_b0 += (valid && (key[e] >> 20) == b0) ? 1u : 0u;
  }
  // Both counts in one scan: each is at most kSelSlice = 4,096 over the
  // block, so they share a word without carries.
  uint32_t both;
  const uint32_t pre2 = block_prefix_sum(keep | (in_b0 << 16), L.scratch, &both);
  uint32_t pos = pre2 & 0xFFFFu;
  const uint32_t total = both & 0xFFFFu, total_b0 = both >> 16;
#pragma unroll
  for (int e = 0; e < kFiltPer; ++e)
    if (j0 + e < g.pe && (key[e] >> 20) >= b0) list_s[pos++] = make_uint2(key[e], (uint32_t)(j0 + e));
  if (threadIdx.x == 0) cnt_r[s] = total;
  if (s == 0 && threadIdx.x == 0) {
    meta_r[0] = b0;
    meta_r[1] = L.res[1];  // pool keys above bin b0
  }
  // Second level: key bits 19..8 of this slice's keys in the threshold bin.
  uint32_t* g2 = hrow + kSelBins;
  if (total_b0 <= kDirectHist2) {
#pragma unroll
    for (int e = 0; e < kFiltPer; ++e)
      if (j0 + e < g.pe && (key[e] >> 20) == b0) atomicAdd(&g2[(key[e] >> 8) & 0xFFFu], 1u);
  } else {
    for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) L.h2[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kFiltPer; ++e)
      if (j0 + e < g.pe && (key[e] >> 20) == b0) atomicAdd(&L.h2[(key[e] >> 8) & 0xFFFu], 1u);
    __syncthreads();
    for (int i = threadIdx.x; i < kSelBins; i += blockDim.x)
      if (L.h2[i] != 0u) atomicAdd(&g2[i], L.h2[i]);
  }
}

constexpr int kMaxSlices = 1024;  // pools up to 4,194,304 keys
constexpr int kStage = 8192;      // list entries held in LDS by the final selection

// LDS of the final selection of one row.
struct FinalLds {
  uint32_t* h;           // [256], 16-byte aligned: key bits 7..0
  uint32_t* pre;         // [kMaxSlices + 1] slice offsets
  uint32_t* chunk_wins;  // [2 * kStage / 64]: per chunk, candidates above and at the threshold
  uint32_t* scratch;     // [16], 16-byte aligned
  uint32_t* res;         // [6]: two result pairs, then the long-slice flag
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
  uint32_t* h = L.h;
  uint32_t* pre = L.pre;
  uint32_t* chunk_wins = L.chunk_wins;
  uint32_t* scratch = L.scratch;
  uint32_t* res_b = L.res;
  uint32_t* res_c = L.res + 2;
  uint2* stage = L.stage;
  const int lane = t & 63, wave = t >> 6;
  const uint2* lr = list + (size_t)r * nslices * kSelSlice;

  // Everything that does not depend on another load is fetched at once,
  // before the row geometry (which waits for the sequence length) is used:
  // the threshold bin b0 that sel_filter found, the second-level histogram
  // (bins kBinsPer t .. kBinsPer t + kBinsPer - 1 per thread), the first 64
  // slice counts, and the head of each slice list this wave will copy first
  // (slices wave + kWaves u for u < kHeads, entries 0..63).  Slices past the
  // row's pool are in the buffers too; their values are not used.
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
  // Wave 0's slice counts, 64 per chunk, for every chunk the buffers hold
  // (issued before the heads: the offsets scan waits for these only).
  constexpr int kCntChunks = kMaxSlices / 64;
  uint32_t cntv[kCntChunks];
#pragma unroll
  for (int c = 0; c < kCntChunks; ++c)
    cntv[c] = (wave == 0 && 64 * c + lane < nslices) ? cnt[(size_t)r * nslices + 64 * c + lane] : 0u;
  constexpr int kHeads = 8;
  uint2 head[kHeads];
#pragma unroll
  for (int u = 0; u < kHeads; ++u) {
    const int sl = wave + kWaves * u;
    if (sl < nslices) head[u] = lr[(size_t)sl * kSelSlice + lane];
  }
  if (g.kk == 0 || g.kk == g.pe) {
    for (int i = t; i < k_top; i += blockDim.x) {
      if (out != nullptr) out[i] = i < g.kk ? i : -1;
      if (win != nullptr && i < g.kk) win[i] = i;
    }
    if (win != nullptr) __syncthreads();
    return g.kk;
  }
  const int ns = (g.pe + kSelSlice - 1) / kSelSlice;
  for (int i = t; i < 256; i += kThreads) h[i] = 0u;  // key bits 7..0, counted while staging

  // Slice offsets: one wave scans the counts 64 at a time, and notes whether
  // any slice holds more entries than its list head (res[4]).
  if (wave == 0) {
    uint32_t carry = 0;
    bool big = false;
#pragma unroll
    for (int ci = 0; ci < kCntChunks; ++ci) {
      const int c0 = 64 * ci;
      if (c0 >= ns) break;
      const uint32_t c = (c0 + lane >= ns) ? 0u : cntv[ci];
      big |= __ballot(c > 64u) != 0ull;
      uint32_t incl = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (c0 + lane < ns) pre[c0 + lane] = carry + incl - c;
      carry += __shfl(incl, 63);
    }
    if (lane == 0) {
      pre[ns] = carry;
      L.res[4] = big ? 1u : 0u;
    }
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
    // Slices wave + kWaves u (u < kHeads): their first 64 entries come from
    // the heads loaded above.
#pragma unroll
    for (int u = 0; u < kHeads; ++u) {
      const int sl = wave + kWaves * u;
      if (sl >= ns) break;
      const uint32_t n = pre[sl + 1] - pre[sl];
      if ((uint32_t)lane < n) put(pre[sl] + lane, head[u]);
    }
    // Every other entry (those of the slices after the first kHeads kWaves,
    // and past the 64th of any slice) by its list position, spread over all
    // threads, the loads of all of a thread's entries issued before any is
    // stored; an entry's slice is found by binary search over the slice
    // offsets.  Without long slices only the later slices' entries are
    // visited.
    constexpr int kFirst = kHeads * kWaves;
    const bool big = L.res[4] != 0u;
    if (ns > kFirst || big) {
      constexpr int kPerT = kStage / kThreads;
      const int s_lo = big ? 0 : kFirst;
      const uint32_t p0 = pre[s_lo];
      uint2 e[kPerT];
      bool mine[kPerT];
#pragma unroll
      for (int k = 0; k < kPerT; ++k) {
        const uint32_t i = p0 + t + (uint32_t)(k * kThreads);
        mine[k] = false;
        if (i < total) {
          int lo = s_lo, hi = ns - 1;  // last slice with pre[s] <= i
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= i) lo = mid;
            else hi = mid - 1;
          }
          const uint32_t li = i - pre[lo];
          mine[k] = lo >= kFirst || li >= 64u;  // else its head put it there
          if (mine[k]) e[k] = lr[(size_t)lo * kSelSlice + li];
        }
      }
#pragma unroll
      for (int k = 0; k < kPerT; ++k)
        if (mine[k]) put(p0 + t + (uint32_t)(k * kThreads), e[k]);
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
  const uint32_t tau = (top24 << 8) | b2;
  __syncthreads();

  // Ordered compaction of the winners: every candidate above tau, and of the
  // candidates equal to tau the need2 first ones, which are those of lowest
  // index because the list is in index order (slices in order, each in key
  // order).  A winner's place is the number of winners before it in the
  // list: those above tau, plus min(need2, candidates equal to tau) before
  // it.  A staged list is cut into 64-entry chunks, one lane per entry:
  // ballots count each chunk's candidates above and at tau, one wave scans
  // the chunk counts, and lanes add the lower lanes of their chunk.  A list
  // left in global memory goes through two block prefix sums over runs of
  // consecutive entries.
  uint32_t base;
  if (staged) {
    // Only the list's chunks are visited (each wave takes chunks wave,
    // wave + kWaves, ...); the ballots are taken again for the writes rather
    // than kept per chunk, which would need a register array per possible
    // chunk.
    const int nchunks = (int)((total + 63) / 64);
    uint32_t* chunk_tau = chunk_wins + kStage / 64;
    auto ballots = [&](int ch, uint64_t& ma, uint64_t& mt) {
      const uint32_t e = 64u * ch + lane;
      const bool valid = e < total;
      const uint32_t kx = valid ? stage[e].x : 0u;
      ma = __ballot(valid && kx > tau);
      mt = __ballot(valid && kx == tau);
    };
    for (int ch = wave; ch < nchunks; ch += kWaves) {
      uint64_t ma, mt;
      ballots(ch, ma, mt);
      if (lane == 0) {
        chunk_wins[ch] = (uint32_t)__popcll(ma);
        chunk_tau[ch] = (uint32_t)__popcll(mt);
      }
    }
    __syncthreads();
    // Candidates above and at tau in the chunks before each chunk: one wave
    // scans both counts in place (res_b gets the totals; the earlier results
    // there are consumed).
    if (wave == 0) {
      uint32_t carry_a = 0, carry_t = 0;
      for (int c0 = 0; c0 < nchunks; c0 += 64) {
        const bool in = c0 + lane < nchunks;
        const uint32_t ca = in ? chunk_wins[c0 + lane] : 0u;
        const uint32_t ct = in ? chunk_tau[c0 + lane] : 0u;
        uint32_t ia = ca, it = ct;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t oa = __shfl_up(ia, off), ot = __shfl_up(it, off);
          if (lane >= off) {
            ia += oa;
            it += ot;
          }
        }
        if (in) {
          chunk_wins[c0 + lane] = carry_a + ia - ca;
          chunk_tau[c0 + lane] = carry_t + it - ct;
        }
        carry_a += __shfl(ia, 63);
        carry_t += __shfl(it, 63);
      }
      if (lane == 0) {
        res_b[0] = carry_a;
        res_b[1] = carry_t;
      }
    }
    __syncthreads();
    base = res_b[0] + min(res_b[1], need2);
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int ch = wave; ch < nchunks; ch += kWaves) {
      uint64_t ma, mt;
      ballots(ch, ma, mt);
      const uint32_t a_before = chunk_wins[ch] + (uint32_t)__popcll(ma & lower);
      const uint32_t t_before = chunk_tau[ch] + (uint32_t)__popcll(mt & lower);
      const bool above = (ma >> lane) & 1ull;
      const bool at = ((mt >> lane) & 1ull) && t_before < need2;
      if (above || at) {
        const uint32_t pos = a_before + min(t_before, need2);
        if (pos < (uint32_t)k_top) {
          if (out != nullptr) out[pos] = (int32_t)stage[64u * ch + lane].y;
          if (win != nullptr) win[pos] = (int32_t)stage[64u * ch + lane].y;
        }
      }
    }
  } else {
    const uint32_t per = (total + blockDim.x - 1) / blockDim.x;
    const uint32_t e0 = min(total, t * per), e1 = min(total, e0 + per);
    uint32_t mine_a = 0, mine_t = 0;
    for (uint32_t e = e0; e < e1; ++e) {
      const uint32_t kx = entry(e).x;
      mine_a += kx > tau ? 1u : 0u;
      mine_t += kx == tau ? 1u : 0u;
    }
    uint32_t tot_a, tot_t;
    uint32_t pa = block_prefix_sum(mine_a, scratch, &tot_a);
    uint32_t pt = block_prefix_sum(mine_t, scratch, &tot_t);
    base = tot_a + min(tot_t, need2);
    for (uint32_t e = e0; e < e1; ++e) {
      const uint2 c = entry(e);
      const bool above = c.x > tau, at = c.x == tau && pt < need2;
      if (above || at) {
        const uint32_t pos = pa + min(pt, need2);
        if (pos < (uint32_t)k_top) {
          if (out != nullptr) out[pos] = (int32_t)c.y;
          if (win != nullptr) win[pos] = (int32_t)c.y;
        }
      }
      pa += above ? 1u : 0u;
      pt += c.x == tau ? 1u : 0u;
    }
  }
  if (out != nullptr)
    for (int i = (int)min(base, (uint32_t)k_top) + t; i < k_top; i += blockDim.x) out[i] = -1;
  if (win != nullptr) __syncthreads();
  return (int)min(base, (uint32_t)k_top);
}

}  // namespace
}  // namespace hs2
