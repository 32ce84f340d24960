// KV Bridging projection: [K | V] = H . [W_K | W_V], bf16 in, fp32 accumulate,
// bf16 out (round to nearest even).
//
// In HySparse2 the K and V caches of each cross-decoder full-attention layer
// are learned projections of a self-decoder full-attention layer's hidden
// states, which lets prefill stop after the self-decoder ("HySparse2: How
// Xiaomi Split the Transformer to Fix Agent Prefill Costs", section "The
// Self-Decoder and Cross-Decoder Split", first two equations; "HySparse2:
// Hybrid Sparse Attention with Two-Level KV Sharing", bullet "KV Bridging").
//
// One fused GEMM with N = 2 x 128 so that H, the dominant operand, is read
// once; with M = 1M and d_model = 2048 it moves about 227 flop per byte,
// under the bf16 MFMA ridge, so it is bound by the H stream.
//
// The weights are static parameters, so they are packed once (bridge_pack)
// into the exact order in which the MFMA B operand consumes them: per 32-deep
// stage, per 32-column tile and 16-deep step, 64 lanes x 16 bytes.
//
// A workgroup owns 256 rows x all 256 columns; each of its 4 waves owns 64
// rows (two 32-row tiles) and keeps sixteen 32x32 fp32 accumulators
// (v_mfma_f32_32x32x16_bf16), so every weight operand read from LDS feeds two
// MFMAs.  Both operands reach LDS by direct global-to-LDS loads (16 bytes a
// lane, no registers in between) through a ring of kStages stages: while the
// MFMAs of one stage run, the operands of the next are read from LDS into
// registers and the loads of the two after it, plus a newly issued one, are
// in flight (up to 64 KiB of H per CU).  Each
// stage holds the 16 KiB packed weight slice, shared by the 4 waves, and each
// wave's own 64 x 32 slice of H, which that wave loads row-contiguously (16
// rows x 64 bytes per instruction) with the 16-byte chunks of a row rotated
// by (row / 4) % 4 so that the operand reads are free of bank conflicts.
// Waits are explicit (the compiler does not track loads to LDS): they are
// counted by vmcnt in issue order, so a wave waits until only its younger
// stages are outstanding, and one barrier per stage both publishes the stage
// to all waves and retires the slot that the next load overwrites.  The output tile is staged through LDS
// so that it leaves in 16-byte row stores.
#include "hs2_internal.h"

namespace hs2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWaves = 4;
constexpr int kBM = 64 * kWaves;                 // rows per workgroup
constexpr int kBN = 256;                         // K columns 0..127, V columns 128..255
constexpr int kBK = 32;                          // reduction depth per stage
constexpr int kStages = 4;                       // LDS ring depth
constexpr int kAhead = kStages;                  // stages issued before the first MFMA
constexpr int kHWave = 64 * kBK * 2;             // 4 KiB of H per wave per stage
constexpr int kHLoads = kHWave / 1024;           // 1 KiB loads per wave per stage
constexpr int kWLoads = 4;                       // weight loads per thread (or wave) per stage

// Weight stage layout, [n tile][16-deep step][lane][8 bf16] (the B operand of
// every MFMA is one 1 KiB block, 16 bytes per lane).  Staged through
// registers, 16 bytes of padding follow every 16 lanes so that the transposing
// 4-byte stores spread over the banks; loaded directly, the blocks are dense.
template <bool kDirect>
struct WLayout {
  static constexpr int kGroup = kDirect ? 256 : 272;        // bytes per 16 lanes
  static constexpr int kBlock = 4 * kGroup;                  // bytes per operand block
  static constexpr int kStage = 16 * kBlock;                 // 8 n tiles x 2 steps
  __device__ static int operand(int n, int s, int lane) {
    return (2 * n + s) * kBlock + (lane >> 4) * kGroup + (lane & 15) * 16;
  }
};

template <bool kDirect>
struct Ring {
  static constexpr int kWStage = WLayout<kDirect>::kStage;
  static constexpr int kStageBytes = kWStage + kWaves * kHWave;
  static constexpr int kBytes = kStages * kStageBytes;
};
static_assert(Ring<true>::kBytes >= kBM * kBN * 2 && Ring<false>::kBytes >= kBM * kBN * 2,
              "output tile reuses the ring");

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// 16 bytes from global memory to LDS at lds + 16 * lane.
__device__ __forceinline__ void load_to_lds(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds, 16, 0, 0);
}

template <int kN>
__device__ __forceinline__ void wait_vm() {
  static_assert(kN >= 0 && kN < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((kN & 15) | ((kN >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most kN loads of this wave are in flight and its LDS reads
// and writes are done, then meet the other waves.
template <int kN>
__device__ __forceinline__ void wait_then_barrier() {
  static_assert(kN >= 0 && kN < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((kN & 15) | ((kN >> 4) << 14) | (7 << 4));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Weights of one stage in registers (the path that transposes W itself):
// thread t holds rows k0+2kp and k0+2kp+1 (kp = item % 16) of the 8 columns
// 8 * (item / 16) .. +7, for its two items t and t + 256.
struct WRegs {
  u32x4 lo[2], hi[2];
};

__device__ __forceinline__ void load_w_regs(const uint16_t* w_k, const uint16_t* w_v, int g, int t,
                                            WRegs& r) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int item = t + 256 * p, kp = item & 15, n0 = 8 * (item >> 4);
    const uint16_t* w = (n0 < kHeadDim ? w_k + n0 : w_v + (n0 - kHeadDim)) +
                        (size_t)(kBK * g + 2 * kp) * kHeadDim;
    r.lo[p] = *reinterpret_cast<const u32x4*>(w);
    r.hi[p] = *reinterpret_cast<const u32x4*>(w + kHeadDim);
  }
}

// Element (k, n) of a stage goes to operand block (n / 32, k / 16), lane
// n % 32 + 32 * (k / 8 % 2), position k % 8; rows k and k+1 share a dword.
__device__ __forceinline__ void store_w_regs(uint8_t* wst, int t, const WRegs& r) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int item = t + 256 * p, kp = item & 15, n0 = 8 * (item >> 4);
    const int k = 2 * kp;
    const int s = k >> 4, half = (k >> 3) & 1, e = k & 7;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = n0 + j;
      const uint32_t lo = r.lo[p][j >> 1], hi = r.hi[p][j >> 1];
      const uint32_t v = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
      *reinterpret_cast<uint32_t*>(wst + WLayout<false>::operand(n >> 5, s, (n & 31) + 32 * half) +
                                   2 * e) = v;
    }
  }
}

// Issue the direct loads of stage g: with packed weights, this wave's quarter
// of the weight stage; always, the wave's own 64 rows of H.
template <bool kDirect>
__device__ __forceinline__ void issue_stage(int g, const uint16_t* w_packed,
                                            const uint16_t* const (&hsrc)[kHLoads], int wave,
                                            int lane, uint8_t* slot) {
  if (kDirect) {
    const uint16_t* ws = w_packed + (size_t)g * 8192 + (kWLoads * wave) * 512 + lane * 8;
#pragma unroll
    for (int j = 0; j < kWLoads; ++j) load_to_lds(ws + j * 512, slot + (kWLoads * wave + j) * 1024);
  }
  uint8_t* hs = slot + Ring<kDirect>::kWStage + wave * kHWave;
#pragma unroll
  for (int j = 0; j < kHLoads; ++j) load_to_lds(hsrc[j] + g * kBK, hs + j * 1024);
}

// The A and B operands of one stage: [16-deep step][m tile] and [step][n tile].
struct Operands {
  u32x4 a[2][2], b[2][8];
};

template <bool kDirect>
__device__ __forceinline__ void read_operands(const uint8_t* st, const int (&a_off)[2][2], int lane,
                                              Operands& o) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) o.a[s][mt] = *reinterpret_cast<const u32x4*>(st + a_off[mt][s]);
#pragma unroll
    for (int n = 0; n < 8; ++n)
      o.b[s][n] = *reinterpret_cast<const u32x4*>(st + WLayout<kDirect>::operand(n, s, lane));
  }
}

// Loads issued per wave per stage, in this order: the weight loads (to LDS
// or to registers), then the H loads.
constexpr int kLoadsPerStage = kWLoads + kHLoads;

// Stage `it`, whose operands are in `cur`: wait for stage it+1 (which also
// retires the slot of stage it, read by every wave), refill that slot with
// stage it+kAhead, read the operands of stage it+1 into `next`, and run the
// 32 MFMAs of stage it while those reads are in flight.  Weights staged
// through registers are loaded at stage it+kAhead's issue and written to LDS
// one step later (so `wnext` and `wcur` alternate), after a wait that only
// forces loads which the next step waits for anyway.  Every step issues the
// same loads, so that the wait counts are constants and the step has no
// branch: past the last stage the loads repeat it (cache-resident) into a
// free slot, and the operands read from it are never used.
template <bool kDirect>
__device__ __forceinline__ void bridge_step(int it, int nk, const uint16_t* w_packed,
                                            const uint16_t* w_k, const uint16_t* w_v,
                                            const uint16_t* const (&hsrc)[kHLoads], int t,
                                            int wave, int lane, const int (&a_off)[2][2],
                                            uint8_t* lds, const Operands& cur, Operands& next,
                                            WRegs& wnext, const WRegs& wcur,
                                            f32x16_t (&acc)[2][8], int rot) {
  constexpr int kSB = Ring<kDirect>::kStageBytes;
  // Younger than stage it+1: stages it+2 .. it+kAhead-1.
  wait_then_barrier<(kAhead - 2) * kLoadsPerStage>();
  int g = min(it + kAhead, nk - 1) + rot;  // rot < nk
  if (g >= nk) g -= nk;
  if (!kDirect) load_w_regs(w_k, w_v, g, t, wnext);
  issue_stage<kDirect>(g, w_packed, hsrc, wave, lane, lds + (it % kStages) * kSB);
  read_operands<kDirect>(lds + ((it + 1) % kStages) * kSB, a_off, lane, next);
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        acc[mt][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(cur.a[s][mt]), as_bf16x8(cur.b[s][n]), acc[mt][n], 0, 0, 0);
  if (!kDirect) {
    // wcur holds stage it+kAhead-1; younger: its H loads and stage it+kAhead.
    wait_vm<kHLoads + kLoadsPerStage>();
    store_w_regs(lds + ((it + kAhead - 1) % kStages) * kSB, t, wcur);
  }
}

template <bool kDirect>
__global__ __launch_bounds__(64 * kWaves) void bridge_gemm(const uint16_t* __restrict__ h,
                                                           int64_t ldh,
                                                           const uint16_t* __restrict__ w_packed,
                                                           const uint16_t* __restrict__ w_k,
                                                           const uint16_t* __restrict__ w_v,
                                                           uint16_t* __restrict__ k_out,
                                                           uint16_t* __restrict__ v_out,
                                                           int64_t ld_kv, int M, int d_model) {
  constexpr int kSB = Ring<kDirect>::kStageBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[Ring<kDirect>::kBytes];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  const int m0 = blockIdx.x * kBM + wave * 64;

  // Load j of a stage brings rows 16j + lane/4 of the wave's 64; the lane's
  // 16-byte chunk is (lane % 4) rotated by the row's (row / 4) % 4.
  const uint16_t* hsrc[kHLoads];
#pragma unroll
  for (int j = 0; j < kHLoads; ++j) {
    const int row = 16 * j + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    hsrc[j] = h + (size_t)min(m0 + row, M - 1) * ldh + 8 * chunk;
  }
  // Operand reads: A tile mt, step s -> row 32mt + r32, chunk 2s + hh.
  int a_off[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int row = 32 * mt + r32, chunk = 2 * s + hh;
      a_off[mt][s] = Ring<kDirect>::kWStage + wave * kHWave +
                     16 * (4 * row + (chunk ^ ((row >> 2) & 3)));
    }

  f32x16_t acc[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[mt][n] = (f32x16_t){};

  const int nk = d_model / kBK;  // even: d_model is a multiple of 64
  // Workgroups start their reduction at different k slices (and wrap), so
  // that at any moment they read different columns of their rows: the
  // concurrent requests spread over more memory channels than when every
  // workgroup reads the same 64 bytes of each of its rows.  Stage s of this
  // workgroup is the k slice phys(s).
  const int rot = blockIdx.x % nk;
  auto phys = [&](int s) {
    const int g = min(s, nk - 1) + rot;
    return g >= nk ? g - nk : g;
  };
  WRegs w0, w1;
  if (kDirect) {
#pragma unroll
    for (int g = 0; g < kAhead; ++g)
      issue_stage<true>(phys(g), w_packed, hsrc, wave, lane, lds + g * kSB);
  } else {
    // Same issue order as the steps (weights, then H, per stage).  Stages
    // 0..2 are written to LDS here; stage 3 stays in w1 for the first step.
    static_assert(kAhead == 4, "prologue written for four stages");
    load_w_regs(w_k, w_v, phys(0), t, w0);
    issue_stage<false>(phys(0), w_packed, hsrc, wave, lane, lds);
    load_w_regs(w_k, w_v, phys(1), t, w1);
    issue_stage<false>(phys(1), w_packed, hsrc, wave, lane, lds + kSB);
    wait_vm<kHLoads + kLoadsPerStage>();
    store_w_regs(lds, t, w0);
    wait_vm<kHLoads>();
    store_w_regs(lds + kSB, t, w1);
    load_w_regs(w_k, w_v, phys(2), t, w0);
    issue_stage<false>(phys(2), w_packed, hsrc, wave, lane, lds + 2 * kSB);
    load_w_regs(w_k, w_v, phys(3), t, w1);
    issue_stage<false>(phys(3), w_packed, hsrc, wave, lane, lds + 3 * kSB);
    wait_vm<kHLoads + kLoadsPerStage>();
    store_w_regs(lds + 2 * kSB, t, w0);
  }
  wait_then_barrier<(kAhead - 1) * kLoadsPerStage>();  // stage 0
  Operands o0, o1;
  read_operands<kDirect>(lds, a_off, lane, o0);
  for (int it = 0; it < nk; it += 2) {
    bridge_step<kDirect>(it, nk, w_packed, w_k, w_v, hsrc, t, wave, lane, a_off, lds, o0, o1, w0,
                         w1, acc, rot);
    bridge_step<kDirect>(it + 1, nk, w_packed, w_k, w_v, hsrc, t, wave, lane, a_off, lds, o1, o0,
                         w1, w0, acc, rot);
  }
  wait_then_barrier<0>();  // every wave is done with the ring

  // acc[mt][n][r]: row 32mt + 8(r/4) + 4hh + r%4 of the wave, column 32n + r32.
  // The wave's 64 x 256 bf16 tile (32 KiB) is staged in its own part of the
  // ring, then leaves as 16-byte pieces, two rows per instruction.
  uint16_t* tile = reinterpret_cast<uint16_t*>(lds + wave * 64 * kBN * 2);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        tile[(32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3)) * kBN + 32 * n + r32] =
            f32_to_bf16_rne(acc[mt][n][r]);
  wait_then_barrier<0>();  // the tiles are in LDS
#pragma unroll 4
  for (int it = 0; it < 32; ++it) {
    const int row = 2 * it + (lane >> 5), piece = lane & 31;
    const int m = m0 + row;
    const u32x4 x = *reinterpret_cast<const u32x4*>(&tile[row * kBN + 8 * piece]);
    if (m < M) {
      uint16_t* out = (piece < 16 ? k_out : v_out) + (size_t)m * ld_kv + 8 * (piece & 15);
      *reinterpret_cast<u32x4*>(out) = x;
    }
  }
}

// w_packed[g][nt][s][lane][e] = W[32g + 16s + 8(lane / 32) + e][32nt + lane % 32]
// with W = [W_K | W_V] (d_model x 256): the B operand of stage g, column tile
// nt and 16-deep step s, 16 bytes per lane.
__global__ __launch_bounds__(256) void bridge_pack(const uint16_t* __restrict__ w_k,
                                                   const uint16_t* __restrict__ w_v,
                                                   uint16_t* __restrict__ w_packed, int d_model) {
  const int idx = blockIdx.x * 256 + threadIdx.x;  // (g, nt, s, lane)
  if (idx >= d_model * 32) return;
  const int lane = idx & 63, s = (idx >> 6) & 1, nt = (idx >> 7) & 7, g = idx >> 10;
  const int n = 32 * nt + (lane & 31);
  const int k0 = kBK * g + 16 * s + 8 * (lane >> 5);
  const uint16_t* w = n < kHeadDim ? w_k + n : w_v + (n - kHeadDim);
  uint32_t p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    p[e] = (uint32_t)w[(size_t)(k0 + 2 * e) * kHeadDim] |
           ((uint32_t)w[(size_t)(k0 + 2 * e + 1) * kHeadDim] << 16);
  *reinterpret_cast<u32x4*>(w_packed + (size_t)idx * 8) = (u32x4){p[0], p[1], p[2], p[3]};
}

}  // namespace

hipError_t launch_bridge_pack(const uint16_t* w_k, const uint16_t* w_v, uint16_t* w_packed,
                              int d_model, hipStream_t st) {
  bridge_pack<<<(d_model * 32 + 255) / 256, 256, 0, st>>>(w_k, w_v, w_packed, d_model);
  return hipGetLastError();
}

hipError_t launch_bridge(const uint16_t* h, int64_t ldh, const uint16_t* w_packed,
                         const uint16_t* w_k, const uint16_t* w_v, uint16_t* k_out,
                         uint16_t* v_out, int64_t ld_kv, int M, int d_model, hipStream_t st) {
  const int grid = (M + kBM - 1) / kBM;
  if (w_packed != nullptr)
    bridge_gemm<true><<<grid, 64 * kWaves, 0, st>>>(h, ldh, w_packed, nullptr, nullptr, k_out,
                                                    v_out, ld_kv, M, d_model);
  else
    bridge_gemm<false><<<grid, 64 * kWaves, 0, st>>>(h, ldh, nullptr, w_k, w_v, k_out, v_out,
                                                     ld_kv, M, d_model);
  return hipGetLastError();
}

}  // namespace hs2
