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
//            registers each) streams its share of the sequence's 32-key
//            blocks, computes the 32 x 32 logit tile of every block on
//            v_mfma_f32_32x32x16_bf16 and folds it into per-head (max, sum);
//            the tiles of its last blocks stay on chip, kRegBlocks per wave
//            in registers and kLdsBlocks per wave in LDS;
//   barrier  the workgroup writes its per-head statistics, then waits until
//            every workgroup of its sequence has written theirs;
//   phase 2  it folds the sequence's statistics into L_h, turns the kept tiles
//            into I[j] without touching HBM, re-reads only its blocks that
//            did not fit, and (in the fused decode step) adds the pool
//            scores to the selector's first histogram;
//   filter   (fused decode step only) after a second barrier, when the
//            sequence's scores and first-level histogram are complete, the
//            selector's candidate filter runs on the sequence's 4,096-key
//            slices c, c + nwg, ... (the same code as the filter kernel).
//
// Workgroup c of a sequence with nwg workgroups takes blocks c, c + nwg,
// c + 2 nwg, ... (its four waves in turn), so that at any moment the
// workgroups of a sequence read neighbouring blocks rather than 1 MiB apart;
// measured, this narrows the spread of their finishing times, which the
// barrier turns into waiting.
//
// The barrier is a generation count per sequence in the workspace: at entry a
// workgroup reads the sequence's generation g, after its statistics it sets its
// own 64-bit slot to tag(g + 1), and it polls the sequence's slots until all of
// them hold that tag; workgroup 0 of the sequence then stores g + 1 as the new
// generation.  The second barrier is the same with a second set of slots and
// a second tag.  No counter has to be reset between calls and a fresh workspace
// needs no initialisation: a slot written by an earlier call holds the tag of
// a generation already passed, and the tag is the generation mixed with a
// fixed 64-bit constant, so other data left in the workspace does not pass for
// it either.  The words sit at fixed positions (generation b at word b, slots
// (b, c) at words kOpMaxWg * (1 + 2b) + c and kOpMaxWg * (2 + 2b) + c) for
// every descriptor.  All
// cross-workgroup data goes through write-through stores and coherent loads
// (sc1), so the L2s of the chip's XCDs need no write-back or invalidation.
// Every workgroup of the grid must be resident at once: the grid never has more
// workgroups than the device has CUs, and the LDS use allows one per CU.  Waits
// are bounded in time; a workgroup that gives up writes NaN scores (and
// empty candidate lists for its slices), so a failure is visible rather than
// silent.
//
// Layout of a logit tile (K as the B operand): lane (r32, hh) holds key
// jb + r32 for heads 8*(r/4) + 4*hh + r%4, r = 0..15, so the sum over heads is
// in-lane plus one cross-half add, exactly as in the two-pass kernel.  Per-head
// statistics are kept per lane against a reference maximum that is the same in
// all 32 lanes of a half; the reference moves (with a rescale) only when a
// logit exceeds it by more than 2^6, so almost every logit costs one exp2, and
// the lanes' sums add without rescaling at the end.
#include "score_common.h"
#include "select_core.h"

namespace hs2 {

using namespace score;

namespace {

constexpr int kOpWaves = 4;
constexpr int kOpThreads = 64 * kOpWaves;
// 32-key tiles per wave kept in registers: the most (in pairs) that compile
// without spilling; a bf16 block needs twice the registers of an E4M3 block
// in flight.
constexpr int kOpRegBlocksBf16 = 20;
constexpr int kOpRegBlocksFp8 = 22;
constexpr int kLdsBlocks = 9;   // ... kept in LDS
constexpr float kRefMin = -1e30f;           // reference of a lane that has seen no key
constexpr float kRescale = 64.f;            // binades a logit may exceed its reference
constexpr uint64_t kWaitTicks = 100000000;  // 1 s of the 100 MHz constant clock
constexpr uint64_t kTagMix = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kTagMix2 = 0xC2B2AE3D27D4EB4Full;

__device__ __forceinline__ uint64_t slot_tag(uint64_t gen) { return gen ^ kTagMix; }
__device__ __forceinline__ uint64_t slot_tag2(uint64_t gen) { return gen ^ kTagMix2; }

struct OpLds {
  union {
    float4 tile[kOpWaves][kLdsBlocks][4][64];  // kept logit tiles: 16 floats per lane
    FilterLds filt;                            // the candidate filter, after phase 2
  };
  // Phase 2: the workgroup's histogram of the top 12 bits of its pool scores,
  // two 16-bit counts per word (bin 2w in the low half of word w); a
  // workgroup counts at most 4,096 keys, so no count reaches the high half.
  uint32_t hist16[kSelBins / 2];
  float2 red[16][32];  // per-wave statistics (end of phase 1), fold partials (phase 2)
  float s_L[32];
  uint64_t tag;
  int wflag[2][kOpWaves];  // barrier polling: per-wave verdicts, by iteration parity
};


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

template <bool kFp8, bool kFilter, int kRegBlocks>
__global__ __launch_bounds__(kOpThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
score_onepass(const uint16_t* __restrict__ q, const void* __restrict__ k, int64_t kv_stride,
              const int32_t* __restrict__ ctx_len, int cap, int H, float c2, int nwg, int chunk,
              float* __restrict__ stats, uint64_t* __restrict__ sync, float* __restrict__ scores,
              float* __restrict__ lse_out, uint32_t* __restrict__ hist, int window,
              FilterArgs filt) {
  // The fused step's variant builds the first-level histogram and runs the
  // candidate filter; the plain one writes the scores only.
  constexpr bool kHist = kFilter;
  __shared__ __attribute__((aligned(16))) OpLds S;
  const int b = blockIdx.x / nwg, c = blockIdx.x - b * nwg;
  const int N = clamp_ctx(ctx_len, b, cap);
  const bool any = 32 * c < N;  // workgroup-uniform: its first block holds keys
  const int nbw = chunk / (32 * kOpWaves);  // blocks per wave
  const int nR = nbw - kRegBlocks;          // blocks before the register-kept ones
  const int nS = nR - kLdsBlocks;           // blocks kept nowhere (read again in phase 2)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  uint64_t* const gen_word = sync + b;
  uint64_t* const slots = sync + (size_t)kOpMaxWg * (1 + 2 * b);
  uint64_t* const slots2 = sync + (size_t)kOpMaxWg * (2 + 2 * b);
  float* const out = scores + (size_t)b * cap;
  const RowGeom rg = row_geom(ctx_len, cap, b, 1, 1, 1, filt.k_top, window);
  // Slices of the selector's filter: those of the pool, unless the pool fits
  // the budget (then the final stage takes it whole).
  const int n_filt = (!kFilter || rg.kk == 0 || rg.kk == rg.pe)
                         ? 0 : (rg.pe + kSelSlice - 1) / kSelSlice;
  // After a failed wait: NaN scores for the keys of the filter slices and
  // empty candidate lists for them.
  auto fail_filter = [&]() {
    for (int s = c; s < n_filt; s += nwg) {
      for (int j = s * kSelSlice + threadIdx.x; j < min(rg.pe, (s + 1) * kSelSlice);
           j += kOpThreads)
        out[j] = __builtin_nanf("");
      if (threadIdx.x == 0) filt.cnt[(size_t)b * filt.nslices + s] = 0u;
      if (s == 0 && threadIdx.x == 0) {
        filt.meta[4 * b] = 0u;
        filt.meta[4 * b + 1] = 0u;
      }
    }
  };

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
  // First key of local block i of this wave, and the key row lane r32 loads
  // (clamped into the context, so every load is in bounds; keys at or past N
  // are never folded or stored).
  auto jb_of = [&](int i) { return 32 * ((i * kOpWaves + wave) * nwg + c); };
  auto row_of = [&](int i) { return min(max(jb_of(i) + r32, 0), N - 1); };
  auto live = [&](int i) { return i >= 0 && jb_of(i) < N; };

  // One register set of K, reloaded piece by piece: as soon as an MFMA has
  // taken a 16-byte piece of the current block, the same piece of the block at
  // next_row is loaded into its place, so the next block's loads are in flight
  // while the current one is folded, in the registers of one block.
  u32x4 kc[k_regs<kFp8>()];
  auto logits_roll = [&](int next_row) {
    const u32x4* kp = reinterpret_cast<const u32x4*>(
                          kb + (size_t)next_row * kHeadDim * kv_elem_bytes<kFp8>()) + hh;
    f32x16_t acc = {};
    if constexpr (kFp8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            qreg[2 * i], as_bf16x8(e4m3x8_to_bf16x8(kc[i][0], kc[i][1])), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            qreg[2 * i + 1], as_bf16x8(e4m3x8_to_bf16x8(kc[i][2], kc[i][3])), acc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        kc[i] = kp[2 * i];
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qreg[e], as_bf16x8(kc[e]), acc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        kc[e] = kp[2 * e];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    return acc;
  };

  float mref[16], lsum[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    mref[r] = kRefMin;
    lsum[r] = 0.f;
  }
  // A kept tile holds e = 2^(x - mref) (the terms of the running sums), so
  // that phase 2 needs no exponential: 2^(x - L) = e * 2^(mref - L).  If the
  // references move after the wave has kept tiles (a logit more than 2^6 above
  // them), the kept values no longer share one scale: the wave then reads all
  // its blocks again in phase 2 (late_move, wave-uniform).
  bool kept_any = false, late_move = false;
  auto fold_tile = [&](const f32x16_t& acc, int jb) {
    const bool valid = jb + r32 < N;
    float dx[16];
    bool up = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dx[r] = (valid ? acc[r] * c2 : -INFINITY) - mref[r];
      up |= dx[r] > kRescale;
    }
    if (__builtin_amdgcn_ballot_w64(up) != 0) {  // rare: move the references up
      late_move |= kept_any;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = valid ? acc[r] * c2 : -INFINITY;
        float bm = x;
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) bm = fmaxf(bm, __shfl_xor(bm, o));
        const float mn = fmaxf(mref[r], bm);
        lsum[r] *= fast_exp2(mref[r] - mn);
        mref[r] = mn;
        dx[r] = x - mn;
      }
    }
    f32x16_t e;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      e[r] = fast_exp2(dx[r]);
      lsum[r] += e[r];
    }
    return e;
  };

  // Waves that prefetch block 0 at the end of phase 1: not wave 0, whose
  // waits for its statistics store and for the barrier would wait for those
  // loads too (memory operations complete in order), and not the workgroup
  // that clears the histograms, whose waves wait for their stores before the
  // barrier.
  const bool pre0 = nS > 0 && wave != 0 && !(kHist && c == 0);
  f32x16_t keep[kRegBlocks];
  float4* my_tiles = &S.tile[wave][0][0][0];
  if (any) {
    // ---- phase 1 ------------------------------------------------------------
    // Blocks [0, nR) are folded, the last kLdsBlocks of them kept in LDS; the
    // next kRegBlocks blocks are folded and kept in registers.  In the waves
    // that prefetch (pre0), the last reload fetches block 0, the first to be
    // read again in phase 2, so that its loads are in flight across the
    // barrier.
    load_k_block<kFp8>(kb, row_of(nR > 0 ? 0 : nR), hh, kc);
    for (int i = 0; i < nR; ++i) {
      const f32x16_t acc = logits_roll(row_of(i + 1));
      if (live(i)) {
        const f32x16_t e = fold_tile(acc, jb_of(i));
        const int s = i - nS;
        if (s >= 0) {
          float4* t = my_tiles + s * 4 * 64 + lane;
#pragma unroll
          for (int p = 0; p < 4; ++p)
            t[p * 64] = make_float4(e[4 * p], e[4 * p + 1], e[4 * p + 2], e[4 * p + 3]);
          kept_any = true;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kRegBlocks; ++t) {
      const int i = nR + t;
      const f32x16_t acc = logits_roll(row_of(i + 1 < nbw ? i + 1 : (pre0 ? 0 : i)));
      if (live(i)) {
        keep[t] = fold_tile(acc, jb_of(i));
        kept_any = true;
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
  // The histogram clears are done before the barrier can pass.  (Only that
  // workgroup waits for its memory operations here: elsewhere the prefetch of
  // block 0 may still be in flight.)
  if (kHist && c == 0) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  float* row = stats + ((size_t)b * nwg + c) * 64;
  // A branch the compiler knows to be wave-uniform, so that the other waves
  // jump over the wait below instead of executing it (a wait is a scalar
  // instruction, carried out whatever the lane mask).
  if (__builtin_amdgcn_readfirstlane(wave) == 0) {
    if (threadIdx.x < 16) {
      float2 a = S.red[0][2 * threadIdx.x], bb = S.red[0][2 * threadIdx.x + 1];
#pragma unroll
      for (int w = 1; w < kOpWaves; ++w) {
        merge_ml(a.x, a.y, S.red[w][2 * threadIdx.x].x, S.red[w][2 * threadIdx.x].y);
        merge_ml(bb.x, bb.y, S.red[w][2 * threadIdx.x + 1].x, S.red[w][2 * threadIdx.x + 1].y);
      }
      const float4 val = make_float4(a.x, a.y, bb.x, bb.y);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, val), buffer_rsrc(row, 256),
                                             threadIdx.x * 16, 0, kSc1);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the row is in memory before the slot says so
    if (threadIdx.x == 0)
      __hip_atomic_store(slots + c, slot_tag(S.tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // ---- barrier: every workgroup of the sequence has written its row --------
  const uint64_t tag = S.tag;
  // Thread t checks slot t of sl; each wave posts "all mine arrived" and "past
  // the time limit", and every wave reads the four posts after one barrier
  // (the posts alternate between two rows, so a fast wave's next post cannot
  // overwrite one that a slow wave is still reading).  Returns true when the
  // time limit passed first.
  auto wait_all = [&](const uint64_t* sl, uint64_t expect) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0;; ++it) {
      const bool mine = threadIdx.x >= nwg ||
                        __hip_atomic_load(sl + threadIdx.x, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == expect;
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
      if (all) return false;
      if (any_late) return true;
      __builtin_amdgcn_s_sleep(8);
    }
  };
  {
    const bool timed_out = wait_all(slots, slot_tag(tag));
    if (c == 0 && threadIdx.x == 0)
      __hip_atomic_store(gen_word, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (timed_out) {
      for (int i = 0; i < nbw; ++i)
        if (hh == 0 && jb_of(i) + r32 < N) out[jb_of(i) + r32] = __builtin_nanf("");
      fail_filter();
      return;
    }
  }
  // ---- phase 2 --------------------------------------------------------------
  // Fold the sequence's rows into L_h with coherent loads (the rows come from
  // other CUs of this launch).  Thread t takes 16-byte piece t % 16 (heads
  // 2p, 2p + 1) of rows t / 16, t / 16 + 16, ...; its loads are issued four
  // at a time, then merged.
  {
    const int pc = threadIdx.x & 15, r0 = threadIdx.x >> 4;
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(stats + (size_t)b * nwg * 64, (uint32_t)(nwg * 64 * sizeof(float)));
    float ma = -INFINITY, la = 0.f, mb = -INFINITY, lb = 0.f;
    for (int base = r0; base < nwg; base += 4 * 16) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int cc = base + 16 * u;
        v[u] = cc < nwg ? __builtin_bit_cast(
                              float4, __builtin_amdgcn_raw_buffer_load_b128(
                                          rs, (cc * 64 + 4 * pc) * 4, 0, kSc1))
                        : make_float4(-INFINITY, 0.f, -INFINITY, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        merge_ml(ma, la, v[u].x, v[u].y);
        merge_ml(mb, lb, v[u].z, v[u].w);
      }
    }
    // 16 partials per head pair: in LDS, then one thread per head.
    float2 (*part)[32] = S.red;  // reused as [16 row groups][16 pieces] of two heads
    reinterpret_cast<float4*>(&part[0][0])[r0 * 16 + pc] = make_float4(ma, la, mb, lb);
    __syncthreads();
    if (threadIdx.x < 32) {
      const int h = threadIdx.x, p = h >> 1, second = h & 1;
      float m = -INFINITY, l = 0.f;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float4 v = reinterpret_cast<const float4*>(&part[0][0])[rr * 16 + p];
        merge_ml(m, l, second ? v.z : v.x, second ? v.w : v.y);
      }
      const float L = (l > 0.f) ? m + log2f(l) : -INFINITY;
      S.s_L[h] = (h < H) ? L : INFINITY;  // padded heads contribute 2^-inf = 0
      if (lse_out != nullptr && c == 0 && h < H) lse_out[b * H + h] = L * 0.69314718055994531f;
    }
    __syncthreads();
  }
  // Scores, and the histogram of the pool ones, of this workgroup's keys.
  auto phase2 = [&]() {
  if (!any) return;  // workgroup-uniform
  float L[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) L[r] = S.s_L[8 * (r >> 2) + 4 * hh + (r & 3)];
  const int pe = N - window;  // decode pool end
  // With the filter, the scores are read by other workgroups of this launch:
  // written through at device scope.
  const __amdgpu_buffer_rsrc_t rs_out = buffer_rsrc(out, (uint32_t)N * 4u);
  if (kHist) {
    for (int i = threadIdx.x; i < kSelBins / 2; i += kOpThreads) S.hist16[i] = 0u;
    __syncthreads();
  }
  // This lane's half (16 heads) of a key's importance.  From logits (blocks
  // read again): sum_h 2^(x - L_h).
  auto part_logits = [&](const f32x16_t& acc) {
    float imp = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) imp += fast_exp2(acc[r] * c2 - L[r]);
    return imp;
  };
  // From kept terms e = 2^(x - mref): sum_h e * 2^(mref_h - L_h).
  float wt[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) wt[r] = fast_exp2(mref[r] - L[r]);
  auto part_kept = [&](const f32x16_t& e) {
    float imp = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) imp = fmaf(e[r], wt[r], imp);
    return imp;
  };
  // After a late move of the references every block of the wave is read again.
  const int n_re = late_move ? nbw : nS;
  // Scores of two blocks from their halves' partial sums: lanes of half 0
  // store block ia's keys, lanes of half 1 block ib's (ib < 0: none).
  auto emit2 = [&](float pa, float pb, int ia, int ib) {
    const float imp = half_sums2(pa, pb);
    const int i = hh ? ib : ia;
    const int j = jb_of(i) + r32;
    if (i >= 0 && j < N) {
      if (kFilter)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(imp), rs_out, j * 4, 0, kSc1);
      else
        out[j] = imp;
      if (kHist && j < pe) {
        const uint32_t bin = order_key(imp) >> 20;
        atomicAdd(&S.hist16[bin >> 1], 1u << (16 * (bin & 1)));
      }
    }
  };
  // Register-kept tiles first (their registers are then free); then the loads
  // of the next blocks to be read again are issued, and the LDS-kept tiles are
  // turned into scores while they are in flight; then the blocks kept nowhere:
  // block 0 from the registers phase 1 left it in, the early ones, the rest
  // four at a time.  The partial sums of a group of tiles are computed before
  // any of it is stored, so that the tiles' chains overlap.
  static_assert(kRegBlocks % 2 == 0, "register tiles go in pairs");
  if (!late_move) {
    float pk[kRegBlocks];
#pragma unroll
    for (int t = 0; t < kRegBlocks; ++t) pk[t] = part_kept(keep[t]);
#pragma unroll
    for (int t = 0; t < kRegBlocks; t += 2) emit2(pk[t], pk[t + 1], nR + t, nR + t + 1);
  }
  const int from_kc = pre0 ? 1 : 0;  // kc holds block 0
  constexpr int kEarly = 3;
  const int n_early = min(kEarly, n_re - from_kc);
  u32x4 ke[kEarly][k_regs<kFp8>()];
#pragma unroll
  for (int u = 0; u < kEarly; ++u)
    if (u < n_early) load_k_block<kFp8>(kb, row_of(from_kc + u), hh, ke[u]);
  if (!late_move) {
    float pl[kLdsBlocks];
#pragma unroll
    for (int u = 0; u < kLdsBlocks; ++u) {
      const float4* t = my_tiles + u * 4 * 64 + lane;
      f32x16_t acc;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float4 v = t[p * 64];
        acc[4 * p] = v.x;
        acc[4 * p + 1] = v.y;
        acc[4 * p + 2] = v.z;
        acc[4 * p + 3] = v.w;
      }
      pl[u] = part_kept(acc);
    }
#pragma unroll
    for (int u = 0; u < kLdsBlocks; u += 2)
      emit2(pl[u], u + 1 < kLdsBlocks ? pl[u + 1] : pl[u], nS + u,
            u + 1 < kLdsBlocks ? nS + u + 1 : -1);
  }
  // Blocks read again, in order, paired as they come (wave-uniform state).
  float held = 0.f;
  int held_i = -1;
  auto reread = [&](const u32x4(&kr)[k_regs<kFp8>()], int i) {
    f32x16_t acc = {};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qreg[e], k_operand<kFp8>(kr, e), acc, 0, 0, 0);
    const float p = part_logits(acc);
    if (held_i < 0) {
      held = p;
      held_i = i;
    } else {
      emit2(held, p, held_i, i);
      held_i = -1;
    }
  };
  if (from_kc) reread(kc, 0);
#pragma unroll
  for (int u = 0; u < kEarly; ++u)
    if (u < n_early) reread(ke[u], from_kc + u);
  for (int i0 = from_kc + kEarly; i0 < n_re; i0 += 4) {
    u32x4 kr[4][k_regs<kFp8>()];
#pragma unroll
    for (int u = 0; u < 4; ++u) load_k_block<kFp8>(kb, row_of(min(i0 + u, n_re - 1)), hh, kr[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (i0 + u >= n_re) break;
      reread(kr[u], i0 + u);
    }
  }
  if (held_i >= 0) emit2(held, held, held_i, -1);
  if (kHist) {
    __syncthreads();
    uint32_t* gh = hist + (size_t)b * kHistRow;
    for (int w = threadIdx.x; w < kSelBins / 2; w += kOpThreads) {
      const uint32_t two = S.hist16[w];
      if (two & 0xFFFFu) atomicAdd(&gh[2 * w], two & 0xFFFFu);
      if (two >> 16) atomicAdd(&gh[2 * w + 1], two >> 16);
    }
  }
  };
  phase2();
  if constexpr (kFilter) {
    // ---- second barrier: the sequence's scores and histogram are complete --
    __builtin_amdgcn_s_waitcnt(0);  // this wave's score stores and atomics are done
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(slots2 + c, slot_tag2(tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (wait_all(slots2, slot_tag2(tag))) {
      fail_filter();
      return;
    }
    // ---- the candidate filter on slices c, c + nwg, ... -----------------------
    uint32_t* hrow = hist + (size_t)b * kHistRow;
    for (int s = c; s < n_filt; s += nwg) {
      uint2* list_s = filt.list + ((size_t)b * filt.nslices + s) * kSelSlice;
      uint32_t* cnt_r = filt.cnt + (size_t)b * filt.nslices;
      if (cap % 4 == 0)
        filter_slice<true, true>(out, cap, rg, s, hrow, cnt_r, filt.meta + 4 * b, list_s, S.filt);
      else
        filter_slice<false, true>(out, cap, rg, s, hrow, cnt_r, filt.meta + 4 * b, list_s, S.filt);
      __syncthreads();
    }
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
                                float* lse, uint32_t* hist, const FilterArgs* filt,
                                hipStream_t st) {
  const auto* qq = static_cast<const uint16_t*>(q);
  const dim3 grid(d.batch * nwg);
  const bool fp8 = d.dtype == HS2_FP8_E4M3;
  FilterArgs fa{};
  fa.k_top = d.k_top;
  const bool fused = filt != nullptr && hist != nullptr;
  if (fused) fa = *filt;
  if (fp8 && fused)
    score_onepass<true, true, kOpRegBlocksFp8><<<grid, kOpThreads, 0, st>>>(
        qq, k, kv_stride, ctx_len, cap, d.n_heads, c2, nwg, chunk, stats, sync, scores, lse, hist,
        d.window, fa);
  else if (fp8)
    score_onepass<true, false, kOpRegBlocksFp8><<<grid, kOpThreads, 0, st>>>(
        qq, k, kv_stride, ctx_len, cap, d.n_heads, c2, nwg, chunk, stats, sync, scores, lse, hist,
        d.window, fa);
  else if (fused)
    score_onepass<false, true, kOpRegBlocksBf16><<<grid, kOpThreads, 0, st>>>(
        qq, k, kv_stride, ctx_len, cap, d.n_heads, c2, nwg, chunk, stats, sync, scores, lse, hist,
        d.window, fa);
  else
    score_onepass<false, false, kOpRegBlocksBf16><<<grid, kOpThreads, 0, st>>>(
        qq, k, kv_stride, ctx_len, cap, d.n_heads, c2, nwg, chunk, stats, sync, scores, lse, hist,
        d.window, fa);
  return hipGetLastError();
}

}  // namespace hs2
