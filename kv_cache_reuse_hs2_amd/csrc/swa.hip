// Sliding-window attention of the self-decoder's SWA layers.
//
// Prefill runs only the self-decoder, whose layers mix full attention with
// sliding-window attention ("HySparse2: How Xiaomi Split the Transformer to
// Fix Agent Prefill Costs", section "The Self-Decoder and Cross-Decoder
// Split").  A query at position P attends to the keys [max(0, P - W + 1), P]
// of one shared K/V head:
//   o_h = sum_j softmax(sm_scale * q_h . k_j) v_j.
//
// Each wave runs a single-pass online softmax for one query over 32-key
// chunks of K and V held in LDS (K rows as they are, 272-byte pitch for
// conflict-free operand reads; V transposed).  QK^T is eight
// v_mfma_f32_32x32x16_bf16 with K as the A operand, so a lane holds one head
// over 16 keys; O is accumulated transposed, O^T += V^T P^T, so the lane that
// holds a head's running max also holds that head's 128 output columns (four
// 32x32 tiles) and the rescaling by 2^(m_old - m_new) needs no data movement.
// The probabilities enter the P.V MFMAs rounded to bf16 (the normaliser is
// summed from the fp32 values), in the key order the QK^T result holds them,
// and the V^T operand is read in that same order.
//
// swa_band_bf16 (windows up to 129 keys): a workgroup takes 32 consecutive
// queries, stages the union of their windows (at most W + 31 keys) into LDS
// once, and each wave then runs four of the queries with no further barrier;
// the next query's Q rows are loaded while the current one computes.  A
// query's whole window (at most five 32-key chunks) is held in registers, so
// its softmax is exact in one step and no accumulator is ever rescaled.
// swa_tiled_bf16 (any window): 8 queries per workgroup, the union of their
// windows streamed through LDS in 64-key tiles.
// V is transposed into LDS two rows at a time (4-byte stores of a key pair,
// consecutive lanes on consecutive words).
#include "hs2_internal.h"

namespace hs2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));

typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Probabilities 8sp .. 8sp + 7 of a lane as the bf16 B operand of a P.V
// step (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ u32x4 bf16_probs(const f32x16_t& p, int sp) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r[j] = __builtin_bit_cast(
        uint32_t, __builtin_convertvector((f32x2_t){p[8 * sp + 2 * j], p[8 * sp + 2 * j + 1]},
                                          bf16x2_t));
  return r;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kSwaWaves = 8;
constexpr int kKPitch = kHeadDim * 2 + 16;  // bytes per staged K row
constexpr float kSlack = 8.f;               // see swa_chunk

// Band kernel: 32 queries, up to 160 staged keys.
constexpr int kBandQ = 32;
constexpr int kBandKeys = 160;
// Transposed V rows: a pitch of w words with gcd(w, 64) = 2 puts the 8-byte
// operand reads of 32 consecutive rows on 32 distinct bank pairs.
constexpr int kBandVt = 164;                // bf16 per transposed V row (82 words)
// Tiled kernel: 8 queries, 64-key tiles.
constexpr int kTileKeys = 64;
constexpr int kTileVt = 68;                 // 34 words

// Output staging: each wave turns its O^T tiles into row-major output rows
// through its own LDS region, so that the global stores are whole 1 KiB
// row segments.  bf16: 32 rows of 256 B; fp32: two passes of 16 rows of
// 512 B; 16 bytes of padding per row spread the 8- and 16-byte writes over
// the banks.
constexpr int kOutPitchB = 256 + 16;   // bf16 output row (bytes)
constexpr int kOutPitchF = 512 + 16;   // fp32 output row (bytes)
constexpr int kOutBytes = 32 * kOutPitchB > 16 * kOutPitchF ? 32 * kOutPitchB : 16 * kOutPitchF;

template <int kKeys, int kVt>
struct SwaLds {
  uint8_t k[kKeys * kKPitch];
  uint16_t vt[kHeadDim][kVt];
  uint8_t out[kSwaWaves][kOutBytes];
};

// The V^T operand of P.V step sp of the chunk at staged row c0, dims
// 32t + r32: keys 16sp + 4hh + 0..3 and 16sp + 8 + 4hh + 0..3, the order in
// which the QK^T result holds the probabilities.
template <int kKeys, int kVt>
__device__ __forceinline__ bf16x8_t v_operand(const SwaLds<kKeys, kVt>& L, int t, int c0, int sp,
                                              int r32, int hh) {
  const uint16_t* vrow = &L.vt[32 * t + r32][c0];
  const uint2 lo4 = *reinterpret_cast<const uint2*>(vrow + 16 * sp + 4 * hh);
  const uint2 hi4 = *reinterpret_cast<const uint2*>(vrow + 16 * sp + 8 + 4 * hh);
  return as_bf16x8((u32x4){lo4.x, lo4.y, hi4.x, hi4.y});
}

struct SwaState {
  float m, l;         // lane: head r32; l over this lane half's keys
  f32x16_t o[4];      // O^T tiles: dims 32t + 8(r/4) + 4hh + r%4, head r32
};

__device__ __forceinline__ void load_q_rows(const uint16_t* qrow, int H, bool live, int r32,
                                            int hh, bf16x8_t (&qr)[8]) {
  // Every lane loads (padded heads repeat head H - 1) and zeroes afterwards:
  // a load under a branch makes the compiler wait for all loads in flight,
  // this one included, at the next use of any earlier load.
  const bool use = live && r32 < H;
  const uint16_t* src = qrow + min(r32, H - 1) * kHeadDim;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    u32x4 x = *reinterpret_cast<const u32x4*>(src + step_dim<false>(e, hh));
    if (!use) x = (u32x4){0u, 0u, 0u, 0u};
    qr[e] = as_bf16x8(x);
  }
}

// Stage keys [key0, key0 + nrows) of the sequence (rows past `last` repeat
// it) into LDS: K rows at row r, V transposed into vt[d][r].  nrows is even
// and at most kKeys.  All of a thread's loads are issued before its first
// LDS store, so the staging costs one memory latency.
template <int kKeys, int kVt, int kThreads>
__device__ __forceinline__ void stage_band(SwaLds<kKeys, kVt>& L, const uint16_t* kb,
                                           const uint16_t* vb, int key0, int last, int nrows) {
  constexpr int kKIt = (kKeys * 16 + kThreads - 1) / kThreads;
  constexpr int kVIt = (kKeys / 2 * 16 + kThreads - 1) / kThreads;
  const int npairs = nrows >> 1;
  u32x4 kx[kKIt], v0[kVIt], v1[kVIt];
#pragma unroll
  for (int it = 0; it < kKIt; ++it) {
    const int e = threadIdx.x + it * kThreads;
    if (e < nrows * 16) {
      const int r = e >> 4, c = e & 15;
      kx[it] = *reinterpret_cast<const u32x4*>(kb + (size_t)min(key0 + r, last) * kHeadDim + 8 * c);
    }
  }
#pragma unroll
  for (int it = 0; it < kVIt; ++it) {
    const int e = threadIdx.x + it * kThreads;
    if (e < npairs * 16) {
      const int p = e % npairs, c = e / npairs;
      v0[it] = *reinterpret_cast<const u32x4*>(vb + (size_t)min(key0 + 2 * p, last) * kHeadDim +
                                               8 * c);
      v1[it] = *reinterpret_cast<const u32x4*>(
          vb + (size_t)min(key0 + 2 * p + 1, last) * kHeadDim + 8 * c);
    }
  }
#pragma unroll
  for (int it = 0; it < kKIt; ++it) {
    const int e = threadIdx.x + it * kThreads;
    if (e < nrows * 16)
      *reinterpret_cast<u32x4*>(L.k + (e >> 4) * kKPitch + 16 * (e & 15)) = kx[it];
  }
#pragma unroll
  for (int it = 0; it < kVIt; ++it) {
    const int e = threadIdx.x + it * kThreads;
    if (e < npairs * 16) {
      const int p = e % npairs, c = e / npairs;
      uint32_t* col = reinterpret_cast<uint32_t*>(&L.vt[8 * c][0]) + p;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        col[(2 * u) * (kVt / 2)] = (v0[it][u] & 0xFFFFu) | (v1[it][u] << 16);
        col[(2 * u + 1) * (kVt / 2)] = (v0[it][u] >> 16) | (v1[it][u] & 0xFFFF0000u);
      }
    }
  }
}

// One 32-key chunk for one query, in two parts: swa_qk computes the logits of
// staged rows c0 .. c0 + 31 (keys a0 .. a0 + 31); swa_softmax_pv updates the
// running softmax and O.  With kMask, keys outside [qlo, P] (or rows at or
// past `valid`) are masked (chunks inside the window skip the test).
template <int kKeys, int kVt>
__device__ __forceinline__ f32x16_t swa_qk(const SwaLds<kKeys, kVt>& L, int c0,
                                           const bf16x8_t (&qr)[8], int r32, int hh) {
  f32x16_t s = {};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bf16x8_t kop = as_bf16x8(
        *reinterpret_cast<const u32x4*>(L.k + (c0 + r32) * kKPitch + 32 * e + 16 * hh));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qr[e], s, 0, 0, 0);
  }
  return s;
}

// The rest of a chunk, given its logits s = swa_qk(c0).
template <bool kMask, int kKeys, int kVt>
__device__ __forceinline__ void swa_softmax_pv(const SwaLds<kKeys, kVt>& L, f32x16_t s, int c0,
                                               int a0, int valid, int qlo, int P, float c2,
                                               int r32, int hh, SwaState& st) {
  // s[r]: head r32, key a0 + 8(r/4) + 4hh + r%4 (chunk row kk = key - a0).
  if (kMask) {
    // Visible rows: lo_k <= kk <= hi_k.
    int lo_k = qlo - a0;
    const int hi_k = min(P - a0, valid - 1 - c0);
    uint32_t span = (uint32_t)(hi_k - lo_k);
    if (hi_k < lo_k) {  // nothing visible
      lo_k = 1 << 20;
      span = 0u;
    }
    const int base = 4 * hh - lo_k;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if ((uint32_t)(base + 8 * (r >> 2) + (r & 3)) > span) s[r] = -INFINITY;
  }
  float bm = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) bm = fmaxf(bm, s[r]);
  bm = fmaxf(bm, __shfl_xor(bm, 32)) * c2;  // c2 > 0: max of the scaled logits
  // Exponent base: moves only when a logit exceeds it by more than kSlack
  // (probabilities relative to it stay below 2^kSlack), so the accumulators
  // are rescaled about once per query instead of at every new maximum.
  const bool move = bm > st.m + kSlack;  // always for the first visible keys
  const float m_new = move ? bm : st.m;
  const float alpha = move ? fast_exp2(st.m - m_new) : 1.f;
  if (__any(move)) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[t][r] *= alpha;
  }
  st.m = m_new;
  const float mref = (m_new == -INFINITY) ? 0.f : m_new;  // no visible key yet
  float x[16];
  float ps = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    x[r] = fast_exp2(fmaf(s[r], c2, -mref));
    ps += x[r];
  }
  st.l = st.l * alpha + ps;
  // O^T += V^T P^T over the chunk's two 16-key steps; step s takes the keys
  // of registers 8s..8s+7: {16s + 4hh + 0..3, 16s + 8 + 4hh + 0..3}.
#pragma unroll
  for (int sp = 0; sp < 2; ++sp) {
    f32x16_t xs;
#pragma unroll
    for (int r = 0; r < 16; ++r) xs[r] = x[r];
    const u32x4 pb = bf16_probs(xs, sp);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      st.o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand(L, t, c0, sp, r32, hh),
                                                        as_bf16x8(pb), st.o[t], 0, 0, 0);
  }
}

// Normalise and write one query's output rows [H][128] at orow (bf16 or
// fp32) and its log-sum-exp at lse_row[h] (if not null), through the wave's
// LDS region `stage`.
template <bool kBf16Out>
__device__ __forceinline__ void swa_store(SwaState& st, void* orow, float* lse_row,
                                          uint8_t* stage, int r32, int hh, int H) {
  const int lane = threadIdx.x & 63;
  const float l_tot = st.l + __shfl_xor(st.l, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[t][r] *= inv;
  if (lse_row != nullptr && hh == 0 && r32 < H)
    lse_row[r32] = l_tot > 0.f ? (st.m + __log2f(l_tot)) * kLn2 : -INFINITY;
  // Lane (r32, hh) holds row r32, columns 32t + 8g + 4hh + 0..3.
  if (kBf16Out) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t w0 = __builtin_bit_cast(
            uint32_t, __builtin_convertvector((f32x2_t){st.o[t][4 * g], st.o[t][4 * g + 1]},
                                              bf16x2_t));
        const uint32_t w1 = __builtin_bit_cast(
            uint32_t, __builtin_convertvector((f32x2_t){st.o[t][4 * g + 2], st.o[t][4 * g + 3]},
                                              bf16x2_t));
        *reinterpret_cast<uint2*>(stage + r32 * kOutPitchB + 2 * (32 * t + 8 * g + 4 * hh)) =
            make_uint2(w0, w1);
      }
    __builtin_amdgcn_wave_barrier();
    uint8_t* dst = static_cast<uint8_t*>(orow);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int idx = lane + 64 * it, h = idx >> 4, c = idx & 15;
      const u32x4 x = *reinterpret_cast<const u32x4*>(stage + h * kOutPitchB + 16 * c);
      if (h < H) *reinterpret_cast<u32x4*>(dst + h * 256 + 16 * c) = x;
    }
  } else {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if ((r32 >> 4) == half) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 x = {st.o[t][4 * g], st.o[t][4 * g + 1], st.o[t][4 * g + 2],
                             st.o[t][4 * g + 3]};
            *reinterpret_cast<f32x4*>(stage + (r32 & 15) * kOutPitchF +
                                      4 * (32 * t + 8 * g + 4 * hh)) = x;
          }
      }
      __builtin_amdgcn_wave_barrier();
      uint8_t* dst = static_cast<uint8_t*>(orow) + (size_t)16 * half * 512;
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int idx = lane + 64 * it, h = idx >> 5, c = idx & 31;
        const u32x4 x = *reinterpret_cast<const u32x4*>(stage + h * kOutPitchF + 16 * c);
        if (16 * half + h < H) *reinterpret_cast<u32x4*>(dst + h * 512 + 16 * c) = x;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

__device__ __forceinline__ void swa_reset(SwaState& st) {
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) st.o[t] = f32x16_t{};
}

// One query of the band kernel: its window touches nch (1..5) consecutive
// 32-row chunks from staged row cf (key a_first).  All its logits stay in
// registers: QK^T of every chunk first (independent accumulators, so the
// MFMAs issue back to back), one exact softmax (no running rescale), then
// P.V.  Only the first and last chunk can hold keys outside [qlo, P].
constexpr int kWinChunks = 5;

__device__ __forceinline__ void swa_window_query(const SwaLds<kBandKeys, kBandVt>& L, int cf,
                                                 int nch, int a_first, int qlo, int P,
                                                 const bf16x8_t (&qr)[8], float c2, int r32,
                                                 int hh, SwaState& st) {
  f32x16_t s[kWinChunks];
#pragma unroll
  for (int c = 0; c < kWinChunks; ++c)
    if (c < nch) s[c] = swa_qk(L, cf + 32 * c, qr, r32, hh);
  float bm = -INFINITY;
#pragma unroll
  for (int c = 0; c < kWinChunks; ++c) {
    if (c >= nch) continue;
    if (c == 0 || c == nch - 1) {
      // Visible rows kk of this chunk: lo_k <= kk <= hi_k.
      const int a0 = a_first + 32 * c;
      const int lo_k = qlo - a0;
      const uint32_t span = (uint32_t)(min(P - a0, 31) - lo_k);
      const int base = 4 * hh - lo_k;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if ((uint32_t)(base + 8 * (r >> 2) + (r & 3)) > span) s[c][r] = -INFINITY;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) bm = fmaxf(bm, s[c][r]);
  }
  bm = fmaxf(bm, __shfl_xor(bm, 32)) * c2;  // c2 > 0: max of the scaled logits
  const float mref = (bm == -INFINITY) ? 0.f : bm;
  float ps = 0.f;
#pragma unroll
  for (int c = 0; c < kWinChunks; ++c) {
    if (c >= nch) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[c][r] = fast_exp2(fmaf(s[c][r], c2, -mref));
      ps += s[c][r];
    }
  }
  st.m = bm;
  st.l = ps;
#pragma unroll
  for (int c = 0; c < kWinChunks; ++c) {
    if (c >= nch) continue;
    const int c0 = cf + 32 * c;
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      const u32x4 pb = bf16_probs(s[c], sp);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        st.o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand(L, t, c0, sp, r32, hh),
                                                          as_bf16x8(pb), st.o[t], 0, 0, 0);
    }
  }
}

// Windows of at most kBandKeys - kBandQ + 1 keys.
template <bool kBf16Out>
__global__ __launch_bounds__(64 * kSwaWaves) void swa_band_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t kv_stride, const int32_t* __restrict__ ctx_len,
    int cap, int n_q, int H, int window, float c2, void* __restrict__ o,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) SwaLds<kBandKeys, kBandVt> L;
  const int b = blockIdx.y, i0 = blockIdx.x * kBandQ;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  const int N = clamp_ctx(ctx_len, b, cap);
  const int p_first = N - n_q + i0, p_last = N - n_q + min(i0 + kBandQ, n_q) - 1;
  const int lo = max(0, p_first - window + 1);
  const int nb = p_last >= 0 ? p_last - lo + 1 : 0;  // <= kBandKeys
  const uint16_t* qb = q + (size_t)b * n_q * H * kHeadDim;

  // This wave's queries: i0 + wave + 8j.  Q rows of the first one load while
  // the band is staged.
  bf16x8_t qr[8], qn[8];
  auto q_of = [&](int j, bf16x8_t(&dst)[8]) {
    const int i = i0 + wave + kSwaWaves * j;
    load_q_rows(qb + (size_t)min(i, n_q - 1) * H * kHeadDim, H, i < n_q && N - n_q + i >= 0, r32,
                hh, dst);
  };
  q_of(0, qr);
  if (nb > 0)
    stage_band<kBandKeys, kBandVt, 64 * kSwaWaves>(L, k + (size_t)b * kv_stride,
                                                   v + (size_t)b * kv_stride, lo, p_last,
                                                   (nb + 31) & ~31);
  __syncthreads();
  for (int j = 0; j < kBandQ / kSwaWaves; ++j) {
    const int i = i0 + wave + kSwaWaves * j;
    if (i >= n_q) break;
    if (j + 1 < kBandQ / kSwaWaves) q_of(j + 1, qn);
    const int P = N - n_q + i;
    SwaState st;
    swa_reset(st);
    if (P >= 0) {
      const int qlo = max(0, P - window + 1);
      const int cf = (qlo - lo) & ~31;
      const int nch = ((P - lo) >> 5) - (cf >> 5) + 1;
      swa_window_query(L, cf, nch, lo + cf, qlo, P, qr, c2, r32, hh, st);
    }
    const size_t row0 = ((size_t)b * n_q + i) * H;
    swa_store<kBf16Out>(st, static_cast<char*>(o) + row0 * kHeadDim * (kBf16Out ? 2 : 4),
                        lse != nullptr ? lse + row0 : nullptr, L.out[wave], r32, hh, H);
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[e] = qn[e];
  }
}

// Any window: 8 queries per workgroup, band streamed in 64-key tiles.
template <bool kBf16Out>
__global__ __launch_bounds__(64 * kSwaWaves) void swa_tiled_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t kv_stride, const int32_t* __restrict__ ctx_len,
    int cap, int n_q, int H, int window, float c2, void* __restrict__ o,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) SwaLds<kTileKeys, kTileVt> L;
  const int b = blockIdx.y, i0 = blockIdx.x * kSwaWaves;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  const int N = clamp_ctx(ctx_len, b, cap);
  const int i = i0 + wave;  // this wave's query
  const int P = N - n_q + i;
  const bool live = i < n_q && P >= 0;
  const int qlo = max(0, P - window + 1);
  const int p_first = N - n_q + i0, p_last = N - n_q + min(i0 + kSwaWaves, n_q) - 1;
  const int lo = max(0, p_first - window + 1);
  const int nb = p_last >= 0 ? p_last - lo + 1 : 0;

  bf16x8_t qr[8];
  load_q_rows(q + ((size_t)b * n_q + min(i, n_q - 1)) * H * kHeadDim, H, live, r32, hh, qr);
  SwaState st;
  swa_reset(st);
  for (int t0 = 0; t0 < nb; t0 += kTileKeys) {
    __syncthreads();  // the previous tile is no longer read
    stage_band<kTileKeys, kTileVt, 64 * kSwaWaves>(L, k + (size_t)b * kv_stride,
                                                   v + (size_t)b * kv_stride, lo + t0, p_last,
                                                   kTileKeys);
    __syncthreads();
    const int kt = min(kTileKeys, nb - t0);
    for (int c0 = 0; c0 < kt; c0 += 32) {
      const int a0 = lo + t0 + c0;
      if (!live || a0 > P || a0 + 31 < qlo) continue;  // chunk outside this window
      const f32x16_t s = swa_qk(L, c0, qr, r32, hh);
      if (a0 < qlo || a0 + 31 > P || c0 + 32 > kt)
        swa_softmax_pv<true>(L, s, c0, a0, kt, qlo, P, c2, r32, hh, st);
      else
        swa_softmax_pv<false>(L, s, c0, a0, kt, qlo, P, c2, r32, hh, st);
    }
  }
  if (i >= n_q) return;
  const size_t row0 = ((size_t)b * n_q + i) * H;
  swa_store<kBf16Out>(st, static_cast<char*>(o) + row0 * kHeadDim * (kBf16Out ? 2 : 4),
                      lse != nullptr ? lse + row0 : nullptr, L.out[wave], r32, hh, H);
}

}  // namespace

hipError_t launch_swa(const hs2_attn_desc& d, const void* q, const void* k, const void* v,
                      int64_t kv_stride, const int32_t* ctx_len, int cap, void* o,
                      bool bf16_out, float* lse, hipStream_t st) {
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  const float c2 = d.sm_scale * kLog2e;
  const dim3 gb((d.n_q + kBandQ - 1) / kBandQ, d.batch);
  const dim3 gt((d.n_q + kSwaWaves - 1) / kSwaWaves, d.batch);
  const bool band = d.window <= kBandKeys - kBandQ + 1;
#define HS2_SWA(KERNEL, GRID, OUT)                                                          \
  KERNEL<OUT><<<GRID, 64 * kSwaWaves, 0, st>>>(qq, kk, vv, kv_stride, ctx_len, cap, d.n_q,   \
                                               d.n_heads, d.window, c2, o, lse)
  if (band && bf16_out)
    HS2_SWA(swa_band_bf16, gb, true);
  else if (band)
    HS2_SWA(swa_band_bf16, gb, false);
  else if (bf16_out)
    HS2_SWA(swa_tiled_bf16, gt, true);
  else
    HS2_SWA(swa_tiled_bf16, gt, false);
#undef HS2_SWA
  return hipGetLastError();
}

}  // namespace hs2
