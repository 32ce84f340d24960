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
// One fused GEMM with N = 2 x 128 so that H (the dominant operand) is read
// once.  A workgroup owns 128 rows x all 256 columns; each of its 4 waves
// owns 32 rows and accumulates eight 32x32 fp32 tiles with
// v_mfma_f32_32x32x16_bf16.  H rows feed the MFMA A operand straight from
// HBM (a lane reads 16 contiguous bytes of one row).  The weights, which
// every workgroup re-reads from L2, are staged per 64-deep K slice into LDS
// transposed ([n][k], k contiguous) as bf16 pairs, so the B operand is one
// 16-byte LDS read per lane; the row pitch of 36 dwords keeps both the
// staging writes and the operand reads free of bank conflicts.
#include "hs2_internal.h"

namespace hs2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int kBM = 128;         // rows per workgroup
constexpr int kBN = 256;         // K columns 0..127, V columns 128..255
constexpr int kBK = 64;          // reduction depth per LDS stage
constexpr int kPitch = kBK / 2 + 4;  // dwords per transposed weight row

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__global__ __launch_bounds__(256) void bridge_gemm(const uint16_t* __restrict__ h, int64_t ldh,
                                                   const uint16_t* __restrict__ w_k,
                                                   const uint16_t* __restrict__ w_v,
                                                   uint16_t* __restrict__ k_out,
                                                   uint16_t* __restrict__ v_out, int64_t ld_kv,
                                                   int M, int d_model) {
  __shared__ uint32_t wt[kBN * kPitch];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  const int m0 = blockIdx.x * kBM + wave * 32;
  const int row = min(m0 + r32, M - 1);
  const uint16_t* hrow = h + (size_t)row * ldh + 8 * hh;

  f32x16_t acc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) acc[n] = (f32x16_t){};

  // Staging assignment: lane -> k pair (t % 32), n block of 8 (t / 32 + 8 * pass).
  const int kp = t & 31, nb = t >> 5;

  u32x4 a[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) a[s] = *reinterpret_cast<const u32x4*>(hrow + 16 * s);

  for (int k0 = 0; k0 < d_model; k0 += kBK) {
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int n0 = (nb + 8 * pass) * 8;  // 0..248
      const uint16_t* w = n0 < 128 ? w_k : w_v;
      const int nc = n0 & 127;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(w + (size_t)(k0 + 2 * kp) * kHeadDim + nc);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(w + (size_t)(k0 + 2 * kp + 1) * kHeadDim + nc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // element 2e and 2e+1 of the 8 columns, paired with the next k row
        wt[(n0 + 2 * e) * kPitch + kp] = (lo[e] & 0xFFFFu) | (hi[e] << 16);
        wt[(n0 + 2 * e + 1) * kPitch + kp] = (lo[e] >> 16) | (hi[e] & 0xFFFF0000u);
      }
    }
    __syncthreads();
    u32x4 an[4];
    const bool more = k0 + kBK < d_model;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if (more) an[s] = *reinterpret_cast<const u32x4*>(hrow + k0 + kBK + 16 * s);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(&wt[(n * 32 + r32) * kPitch + 8 * s + 4 * hh]);
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[s]), as_bf16x8(b), acc[n], 0, 0, 0);
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = an[s];
  }
  // acc[n][r]: row m0 + 8*(r/4) + 4*hh + r%4, column 32*n + r32.
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    uint16_t* out = n < 4 ? k_out : v_out;
    const int col = (n & 3) * 32 + r32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (m < M) out[(size_t)m * ld_kv + col] = f32_to_bf16_rne(acc[n][r]);
    }
  }
}

}  // namespace

hipError_t launch_bridge(const uint16_t* h, int64_t ldh, const uint16_t* w_k, const uint16_t* w_v,
                         uint16_t* k_out, uint16_t* v_out, int64_t ld_kv, int M, int d_model,
                         hipStream_t st) {
  const int grid = (M + kBM - 1) / kBM;
  bridge_gemm<<<grid, 256, 0, st>>>(h, ldh, w_k, w_v, k_out, v_out, ld_kv, M, d_model);
  return hipGetLastError();
}

}  // namespace hs2
