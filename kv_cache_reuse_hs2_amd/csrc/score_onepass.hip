// Full-attention scoring for a decode step in one pass over the K cache.
//
// The full layer's attention over the whole context yields the per-key
// importance that the selection is made from ("HySparse2: How Xiaomi Split
// the Transformer to Fix Agent Prefill Costs", section "KV Reuse and
// Token-Level Sparse Selection"):
//   I[j] = sum_h 2^(x_hj - L_h),  x_hj = (sm_scale*log2 e) * q_h.k_j,
//   L_h  = log2 sum_j 2^(x_hj).
// L_h depends on every key, so an exact I[j] for any key needs either a second
// read of K or the logits of every key kept until L_h is known.  At the decode
// shapes here the logits fit on chip: 32 fp32 logits per key are 128 B, and a
// CU holds 512 KiB of registers and 160 KiB of LDS.  So this kernel reads K
// once:
//
//   phase 1  each workgroup (one per CU, four waves, one per SIMD with 512
//            registers each) streams its chunk of the sequence's keys,
//            computes the 32 x 32 logit tile of every 32-key block on
//            v_mfma_f32_32x32x16_bf16 and folds it into per-head (max, sum);
//            the tiles of the chunk's last blocks stay on chip, kRegBlocks
//            per wave in registers and kLdsBlocks per wave in LDS;
//   barrier  the workgroup writes its per-head statistics, then waits until
//            every workgroup of its sequence has written theirs;
//   phase 2  it folds the sequence's statistics into L_h, turns the kept tiles
//            into I[j] without touching HBM, re-reads only the keys of its
//            chunk that did not fit, and (in the fused decode step) adds the
//            pool scores to the selector's first histogram.
//
// The barrier is a generation count per sequence in the workspace: at entry a
// workgroup reads the sequence's generation g, after its statistics it sets its
// own 64-bit slot to tag(g + 1), and it polls the sequence's slots until all of
// them hold that tag; workgroup 0 of the sequence then stores g + 1 as the new
// generation.  No counter has to be reset between calls and a fresh workspace
// needs no initialisation: a slot written by an earlier call holds the tag of
// a generation already passed, and the tag is the generation mixed with a
// fixed 64-bit constant, so other data left in the workspace does not pass for
// it either.  The words sit at fixed positions (generation b at word b, slot
// (b, c) at word kOpMaxWg * (1 + b) + c) for every descriptor.  All
// cross-workgroup data goes through write-through stores and coherent loads
// (sc1), so the L2s of the chip's XCDs need no write-back or invalidation.
// Every workgroup of the grid must be resident at once: the grid never has more
// workgroups than the device has CUs, and the LDS use allows one per CU.  Waits
// are bounded in time; a workgroup that gives up writes NaN scores, so a
// failure is visible rather than silent.
//
// Layout of a logit tile (K as the B operand): lane (r32, hh) holds key
// jb + r32 for heads 8*(r/4) + 4*hh + r%4, r = 0..15, so the sum over heads is
// in-lane plus one cross-half add, exactly as in the two-pass kernel.  Per-head
// statistics are kept per lane against a reference maximum that is the same in
// all 32 lanes of a half; the reference moves (with a rescale) only when a
// logit exceeds it by more than 2^6, so almost every logit costs one exp2, and
// the lanes' sums add without rescaling at the end.
#include "score_common.h"

namespace hs2 {

using namespace score;

namespace {

constexpr int kOpWaves = 4;
constexpr int kOpThreads = 64 * kOpWaves;
constexpr int kRegBlocks = 16;  // 32-key tiles per wave kept in registers (even)
constexpr int kLdsBlocks = 9;   // ... kept in LDS
constexpr float kRefMin = -1e30f;           // reference of a lane that has seen no key
constexpr float kRescale = 64.f;            // binades a logit may exceed its reference
constexpr uint64_t kWaitTicks = 100000000;  // 1 s of the 100 MHz constant clock
constexpr uint64_t kTagMix = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t slot_tag(uint64_t gen) { return gen ^ kTagMix; }

struct OpLds {
  union {
    float4 tile[kOpWaves][kLdsBlocks][4][64];  // kept logit tiles: 16 floats per lane
    uint32_t hist[kSelBins];                   // phase 2, once the tiles are read
  } u;
  float2 red[8][32];  // per-wave statistics (end of phase 1), fold partials (phase 2)
  float s_L[32];
  uint64_t tag;
  int wflag[2][kOpWaves];  // barrier polling: per-wave verdicts, by iteration parity
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
constexpr int kSc1 = 16;  // cache policy: coherent at device scope (sc1)

// a if c else b, as a bit select (an indexed form would make the compiler put
// the arrays below in memory).
__device__ __forceinline__ float pick(bool c, float a, float b) {
  const uint32_t m = 0u - static_cast<uint32_t>(c);
  return __uint_as_float((__float_as_uint(a) & m) | (__float_as_uint(b) & ~m));
}

// Reduce-scatter of sixteen per-lane values over the 32 lanes of a half:
// afterwards lane r32 holds, for slot s = r32 >> 1, the sum of v[s] over the
// half, and the (half-uniform) m[s].
__device__ __forceinline__ void half_reduce_scatter(const float (&v)[16], const float (&m)[16],
                                                    int r32, float& out_v, float& out_m) {
  float v8[8], m8[8];
  const bool b4 = (r32 >> 4) & 1;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    v8[k] = pick(b4, v[k + 8], v[k]) + __shfl_xor(pick(b4, v[k], v[k + 8]), 16);
    m8[k] = pick(b4, m[k + 8], m[k]);
  }
  float v4[4], m4[4];
  const bool b3 = (r32 >> 3) & 1;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v4[k] = pick(b3, v8[k + 4], v8[k]) + __shfl_xor(pick(b3, v8[k], v8[k + 4]), 8);
    m4[k] = pick(b3, m8[k + 4], m8[k]);
  }
  float v2[2], m2[2];
  const bool b2 = (r32 >> 2) & 1;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    v2[k] = pick(b2, v4[k + 2], v4[k]) + __shfl_xor(pick(b2, v4[k], v4[k + 2]), 4);
    m2[k] = pick(b2, m4[k + 2], m4[k]);
  }
  const bool b1 = (r32 >> 1) & 1;
  out_v = pick(b1, v2[1], v2[0]) + __shfl_xor(pick(b1, v2[0], v2[1]), 2);
  out_m = pick(b1, m2[1], m2[0]);
  out_v += __shfl_xor(out_v, 1);
  // slot s = 8*b4 + 4*b3 + 2*b2 + b1 = r32 >> 1
}

template <bool kFp8, bool kHist>
__global__ __launch_bounds__(kOpThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
score_onepass(const uint16_t* __restrict__ q, const void* __restrict__ k, int64_t kv_stride,
              const int32_t* __restrict__ ctx_len, int cap, int H, float c2, int nwg, int chunk,
              float* __restrict__ stats, uint64_t* __restrict__ sync, float* __restrict__ scores,
              int64_t score_stride, float* __restrict__ lse_out, uint32_t* __restrict__ hist,
              int window) {
  __shared__ __attribute__((aligned(16))) OpLds S;
  const int b = blockIdx.x / nwg, c = blockIdx.x - b * nwg;
  const int N = clamp_ctx(ctx_len, b, cap);
  const int j_begin = c * chunk;
  const int j_end = min(N, j_begin + chunk);
  const bool any = j_begin < j_end;  // workgroup-uniform
  const int nbw = chunk / (32 * kOpWaves);  // blocks per wave (even)
  const int nR = nbw - kRegBlocks;          // blocks before the register-kept ones
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  uint64_t* const gen_word = sync + b;
  uint64_t* const slots = sync + (size_t)kOpMaxWg * (1 + b);

  if (threadIdx.x == 0) {
    const uint64_t g = __hip_atomic_load(gen_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    S.tag = g + 1;
  }
  // The selector histograms of this sequence (both levels; the first is
  // filled after the barrier, the second by the selector's filter) are
  // cleared with write-through stores, which the barrier orders before the
  // other workgroups' atomics.
  if (kHist && c == 0)
    for (int i = threadIdx.x; i < kHistRow; i += kOpThreads)
      __hip_atomic_store(hist + (size_t)b * kHistRow + i, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);

  const char* kb = static_cast<const char*>(k) + (size_t)b * kv_stride * kv_elem_bytes<kFp8>();
  bf16x8_t qreg[8];
  load_q_bf16<kFp8>(q + (size_t)b * H * kHeadDim, H, r32, hh, qreg);
  // Key rows of local block i of this wave (clamped into the context, so every
  // load is in bounds; blocks outside [j_begin, j_end) are never computed).
  auto jb_of = [&](int i) { return j_begin + 32 * (i * kOpWaves + wave); };
  auto row_of = [&](int i) { return min(max(jb_of(i) + r32, 0), N - 1); };
  auto live = [&](int i) { return i >= 0 && jb_of(i) < j_end; };

  float mref[16], lsum[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    mref[r] = kRefMin;
    lsum[r] = 0.f;
  }
  auto logits = [&](const u32x4 (&kc)[k_regs<kFp8>()]) {
    f32x16_t acc = {};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qreg[i], k_operand<kFp8>(kc, i), acc, 0, 0, 0);
    return acc;
  };
  auto fold_tile = [&](const f32x16_t& acc, int jb) {
    const bool valid = jb + r32 < j_end;
    float x[16];
    bool up = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[r] = valid ? acc[r] * c2 : -INFINITY;
      up |= x[r] > mref[r] + kRescale;
    }
    if (__builtin_amdgcn_ballot_w64(up) != 0) {  // rare: move the references up
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float bm = x[r];
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) bm = fmaxf(bm, __shfl_xor(bm, o));
        const float mn = fmaxf(mref[r], bm);
        lsum[r] *= fast_exp2(mref[r] - mn);
        mref[r] = mn;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) lsum[r] += fast_exp2(x[r] - mref[r]);
  };

  f32x16_t keep[kRegBlocks];
  u32x4 ka[k_regs<kFp8>()], kn[k_regs<kFp8>()];
  float4* my_tiles = &S.u.tile[wave][0][0][0];
  if (any) {
    // ---- phase 1 ------------------------------------------------------------
    // Blocks [0, nR): streamed, the last kLdsBlocks of them kept in LDS; then
    // kRegBlocks blocks kept in registers.  Two register sets are used in
    // turn with unconditional loads, so the next block's loads are in flight
    // while the current one is computed.
    load_k_block<kFp8>(kb, row_of(nR > 0 ? 0 : nR), hh, ka);
    auto stream_block = [&](const u32x4 (&kc)[k_regs<kFp8>()], int i) {
      if (!live(i)) return;
      const f32x16_t acc = logits(kc);
      fold_tile(acc, jb_of(i));
      const int s = i - (nR - kLdsBlocks);
      if (s >= 0) {
        float4* t = my_tiles + s * 4 * 64 + lane;
#pragma unroll
        for (int p = 0; p < 4; ++p)
          t[p * 64] = make_float4(acc[4 * p], acc[4 * p + 1], acc[4 * p + 2], acc[4 * p + 3]);
      }
    };
    for (int i = 0; i < nR; i += 2) {
      load_k_block<kFp8>(kb, row_of(i + 1), hh, kn);
      __builtin_amdgcn_sched_barrier(0);
      stream_block(ka, i);
      load_k_block<kFp8>(kb, row_of(i + 2), hh, ka);
      __builtin_amdgcn_sched_barrier(0);
      stream_block(kn, i + 1);
    }
#pragma unroll
    for (int t = 0; t < kRegBlocks; ++t) {
      const int i = nR + t;
      if (t + 1 < kRegBlocks) {
        if (t & 1)
          load_k_block<kFp8>(kb, row_of(i + 1), hh, ka);
        else
          load_k_block<kFp8>(kb, row_of(i + 1), hh, kn);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (live(i)) {
        keep[t] = (t & 1) ? logits(kn) : logits(ka);
        fold_tile(keep[t], jb_of(i));
      }
    }
  }
  // Per-head statistics of the wave: sums over the half's lanes, then the four
  // waves merged, written through to memory.
  {
    float v, m;
    half_reduce_scatter(lsum, mref, r32, v, m);
    const int s = r32 >> 1;
    const int h = 8 * (s >> 2) + 4 * hh + (s & 3);
    if ((r32 & 1) == 0) S.red[wave][h] = make_float2(m, v);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's write-through stores are done
  __syncthreads();
  float* row = stats + ((size_t)b * nwg + c) * 64;
  if (wave == 0) {
    if (threadIdx.x < 16) {
      float2 a = S.red[0][2 * threadIdx.x], bb = S.red[0][2 * threadIdx.x + 1];
#pragma unroll
      for (int w = 1; w < kOpWaves; ++w) {
        merge_ml(a.x, a.y, S.red[w][2 * threadIdx.x].x, S.red[w][2 * threadIdx.x].y);
        merge_ml(bb.x, bb.y, S.red[w][2 * threadIdx.x + 1].x, S.red[w][2 * threadIdx.x + 1].y);
      }
      const float4 val = make_float4(a.x, a.y, bb.x, bb.y);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, val), rsrc_of(row, 256),
                                             threadIdx.x * 16, 0, kSc1);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the row is in memory before the slot says so
    if (threadIdx.x == 0)
      __hip_atomic_store(slots + c, slot_tag(S.tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // ---- barrier: every workgroup of the sequence has written its row --------
  const uint64_t tag = S.tag;
  {
    // Thread t checks slot t; each wave posts "all mine arrived" and "past the
    // time limit", and every wave reads the four posts after one barrier (the
    // posts alternate between two rows, so a fast wave's next post cannot
    // overwrite one that a slow wave is still reading).
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool timed_out = false;
    for (int it = 0;; ++it) {
      const bool mine = threadIdx.x >= nwg ||
                        __hip_atomic_load(slots + threadIdx.x, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == slot_tag(tag);
      const bool late = __builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks;
      const uint64_t missing = __builtin_amdgcn_ballot_w64(!mine);
      const uint64_t over = __builtin_amdgcn_ballot_w64(late);
      if (lane == 0) S.wflag[it & 1][wave] = (missing == 0 ? 1 : 0) | (over != 0 ? 2 : 0);
      __syncthreads();
      int all = 1, any_late = 0;
#pragma unroll
      for (int w = 0; w < kOpWaves; ++w) {
        all &= S.wflag[it & 1][w] & 1;
        any_late |= S.wflag[it & 1][w] & 2;
      }
      if (all) break;
      if (any_late) {
        timed_out = true;
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
    if (c == 0 && threadIdx.x == 0)
      __hip_atomic_store(gen_word, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (timed_out) {
      float* out = scores + (size_t)b * score_stride;
      for (int j = j_begin + threadIdx.x; j < j_end; j += kOpThreads) out[j] = __builtin_nanf("");
      return;
    }
  }
  // ---- phase 2 --------------------------------------------------------------
  // Fold the sequence's rows into L_h (coherent loads: the rows come from other
  // CUs of this launch).
  {
    const int h = threadIdx.x & 31, part = threadIdx.x >> 5;
    const __amdgpu_buffer_rsrc_t rs =
        rsrc_of(stats + (size_t)b * nwg * 64, (uint32_t)(nwg * 64 * sizeof(float)));
    float m = -INFINITY, l = 0.f;
    for (int cc = part; cc < nwg; cc += 8) {
      const float2 v = __builtin_bit_cast(
          float2, __builtin_amdgcn_raw_buffer_load_b64(rs, (cc * 64 + 2 * h) * 4, 0, kSc1));
      merge_ml(m, l, v.x, v.y);
    }
    S.red[part][h] = make_float2(m, l);
    __syncthreads();
    if (threadIdx.x < 32) {
      m = S.red[0][h].x;
      l = S.red[0][h].y;
#pragma unroll
      for (int p = 1; p < 8; ++p) merge_ml(m, l, S.red[p][h].x, S.red[p][h].y);
      const float L = (l > 0.f) ? m + log2f(l) : -INFINITY;
      S.s_L[h] = (h < H) ? L : INFINITY;  // padded heads contribute 2^-inf = 0
      if (lse_out != nullptr && c == 0 && h < H) lse_out[b * H + h] = L * 0.69314718055994531f;
    }
    __syncthreads();
  }
  if (!any) return;  // workgroup-uniform
  float L[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) L[r] = S.s_L[8 * (r >> 2) + 4 * hh + (r & 3)];
  float* out = scores + (size_t)b * score_stride;
  const int pe = N - window;  // decode pool end
  const int nS = nR - kLdsBlocks;  // blocks that were not kept
  // Start re-reading the first block that was not kept.
  if (nS > 0) load_k_block<kFp8>(kb, row_of(0), hh, ka);
  auto importance = [&](const f32x16_t& acc) {
    float imp = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) imp += fast_exp2(acc[r] * c2 - L[r]);
    return imp + __shfl_xor(imp, 32);
  };
  // LDS-kept tiles first (their scores are held until the histogram is free).
  float lds_imp[kLdsBlocks];
#pragma unroll
  for (int s = 0; s < kLdsBlocks; ++s) {
    const int i = nR - kLdsBlocks + s;
    lds_imp[s] = 0.f;
    if (live(i)) {
      const float4* t = my_tiles + s * 4 * 64 + lane;
      f32x16_t acc;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float4 v = t[p * 64];
        acc[4 * p] = v.x;
        acc[4 * p + 1] = v.y;
        acc[4 * p + 2] = v.z;
        acc[4 * p + 3] = v.w;
      }
      lds_imp[s] = importance(acc);
      const int j = jb_of(i) + r32;
      if (hh == 0 && j < j_end) out[j] = lds_imp[s];
    }
  }
  if (kHist) {
    __syncthreads();  // every wave has read its tiles
    for (int i = threadIdx.x; i < kSelBins; i += kOpThreads) S.u.hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kLdsBlocks; ++s) {
      const int i = nR - kLdsBlocks + s;
      const int j = jb_of(i) + r32;
      if (live(i) && hh == 0 && j < j_end && j < pe)
        atomicAdd(&S.u.hist[order_key(lds_imp[s]) >> 20], 1u);
    }
  }
  auto emit = [&](float imp, int jb) {
    const int j = jb + r32;
    if (hh == 0 && j < j_end) {
      out[j] = imp;
      if (kHist && j < pe) atomicAdd(&S.u.hist[order_key(imp) >> 20], 1u);
    }
  };
#pragma unroll
  for (int t = 0; t < kRegBlocks; ++t) {
    const int i = nR + t;
    if (live(i)) emit(importance(keep[t]), jb_of(i));
  }
  // Blocks that did not fit: read again.
  for (int i = 0; i < nS; i += 2) {
    load_k_block<kFp8>(kb, row_of(i + 1 < nS ? i + 1 : i), hh, kn);
    __builtin_amdgcn_sched_barrier(0);
    if (live(i)) emit(importance(logits(ka)), jb_of(i));
    if (i + 1 >= nS) break;
    load_k_block<kFp8>(kb, row_of(i + 2 < nS ? i + 2 : i + 1), hh, ka);
    __builtin_amdgcn_sched_barrier(0);
    if (live(i + 1)) emit(importance(logits(kn)), jb_of(i + 1));
  }
  if (kHist) {
    __syncthreads();
    uint32_t* gh = hist + (size_t)b * kHistRow;
    for (int i = threadIdx.x; i < kSelBins; i += kOpThreads)
      if (S.u.hist[i] != 0u) atomicAdd(&gh[i], S.u.hist[i]);
  }
}

}  // namespace

// Workgroups per sequence and keys per workgroup of the one-pass kernel, or
// false when the batch does not fit the device's CUs.
bool onepass_plan(const hs2_attn_desc& d, int cap, int n_cu, int* nwg, int* chunk) {
  n_cu = min(n_cu, kOpMaxWg);
  if (d.dtype == HS2_F32 || d.batch > n_cu) return false;
  const int per_seq = n_cu / d.batch;
  const int blocks2 = (cap + 255) / 256;  // 256-key units (two blocks per wave)
  const int n = max(1, min(per_seq, blocks2));
  *nwg = n;
  *chunk = ((blocks2 + n - 1) / n) * 256;
  return true;
}

int device_cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev] = n;
  return n;
}

hipError_t launch_score_onepass(const hs2_attn_desc& d, const void* q, const void* k,
                                int64_t kv_stride, const int32_t* ctx_len, int cap, int nwg,
                                int chunk, float c2, float* stats, uint64_t* sync, float* scores,
                                float* lse, uint32_t* hist, hipStream_t st) {
  const auto* qq = static_cast<const uint16_t*>(q);
  const dim3 grid(d.batch * nwg);
  const bool fp8 = d.dtype == HS2_FP8_E4M3;
  if (fp8 && hist)
    score_onepass<true, true><<<grid, kOpThreads, 0, st>>>(qq, k, kv_stride, ctx_len, cap,
                                                           d.n_heads, c2, nwg, chunk, stats, sync,
                                                           scores, cap, lse, hist, d.window);
  else if (fp8)
    score_onepass<true, false><<<grid, kOpThreads, 0, st>>>(qq, k, kv_stride, ctx_len, cap,
                                                            d.n_heads, c2, nwg, chunk, stats,
                                                            sync, scores, cap, lse, hist, d.window);
  else if (hist)
    score_onepass<false, true><<<grid, kOpThreads, 0, st>>>(qq, k, kv_stride, ctx_len, cap,
                                                            d.n_heads, c2, nwg, chunk, stats,
                                                            sync, scores, cap, lse, hist, d.window);
  else
    score_onepass<false, false><<<grid, kOpThreads, 0, st>>>(qq, k, kv_stride, ctx_len, cap,
                                                             d.n_heads, c2, nwg, chunk, stats,
                                                             sync, scores, cap, lse, hist,
                                                             d.window);
  return hipGetLastError();
}

}  // namespace hs2
