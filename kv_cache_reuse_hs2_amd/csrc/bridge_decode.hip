// KV Bridging of one new token per sequence during decode.
//
// The cross-decoder's full-attention K and V are learned projections of a
// self-decoder full-attention layer's hidden states ("HySparse2: How Xiaomi
// Split the Transformer to Fix Agent Prefill Costs", section "The
// Self-Decoder and Cross-Decoder Split", first two equations).  In decode
// each sequence adds one token, so the projection is [B][d_model] x
// [d_model][256] ([W_K | W_V]) and the results go to one cache row per
// sequence.  The work is a few MFMAs per weight byte: the 1 MiB of packed
// weights is the whole cost, so the kernel spreads their reads over many
// waves and keeps every wave's loads in flight together.
//
// Workgroup (nt, rt): columns 32nt .. 32nt + 31 of [K | V] for batch rows
// 32rt .. 32rt + 31, one v_mfma_f32_32x32x16_bf16 per 16-deep k-step.  Its 8
// waves take k-steps w, w + 8, ... (the B operands come straight from the
// packed weights, 16 bytes a lane, in the order hs2_bridge_pack_weights
// stores them), issue all of a batch of 16 steps' loads before the first
// MFMA, and add their partial tiles in LDS in wave order.  One rounding to
// bf16 at the end, as in the bulk projection.
#include "hs2_internal.h"

namespace hs2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

constexpr int kBdWaves = 8;
constexpr int kBdBatch = 16;  // k-steps whose loads a wave issues together

__global__ __launch_bounds__(64 * kBdWaves) void bridge_decode(
    const uint16_t* __restrict__ h, int64_t ldh, const uint16_t* __restrict__ w_packed,
    int rows, int d_model, const int32_t* __restrict__ pos, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache, int64_t kv_stride, int cap) {
  __shared__ float red[kBdWaves][32][33];
  const int nt = blockIdx.x, rt = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  const int row = rt * 32 + r32;
  const bool live = row < rows;
  const uint16_t* hrow = h + (size_t)min(row, rows - 1) * ldh + 8 * hh;
  const int nks = d_model / 16;
  f32x16_t acc = {};
  for (int k0 = wave; k0 < nks; k0 += kBdWaves * kBdBatch) {
    u32x4 a[kBdBatch], b[kBdBatch];
#pragma unroll
    for (int u = 0; u < kBdBatch; ++u) {
      const int kk = k0 + kBdWaves * u;
      a[u] = (u32x4){0u, 0u, 0u, 0u};
      b[u] = (u32x4){0u, 0u, 0u, 0u};
      if (kk < nks) {
        if (live) a[u] = *reinterpret_cast<const u32x4*>(hrow + 16 * kk);
        const size_t idx = ((size_t)((kk >> 1) * 8 + nt) * 2 + (kk & 1)) * 64 + lane;
        b[u] = *reinterpret_cast<const u32x4*>(w_packed + idx * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < kBdBatch; ++u)
      if (k0 + kBdWaves * u < nks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[u]), as_bf16x8(b[u]), acc, 0,
                                                      0, 0);
  }
  // acc[r]: batch row 8(r/4) + 4hh + r%4 of the tile, column r32.
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][8 * (r >> 2) + 4 * hh + (r & 3)][r32] = acc[r];
  __syncthreads();
  for (int e = threadIdx.x; e < 32 * 32; e += blockDim.x) {
    const int tr = e >> 5, col = e & 31;
    const int bq = rt * 32 + tr;
    if (bq >= rows) continue;
    const int p = pos[bq];
    if (p < 0 || p >= cap) continue;
    float sum = red[0][tr][col];
#pragma unroll
    for (int w = 1; w < kBdWaves; ++w) sum += red[w][tr][col];
    const int n = 32 * nt + col;
    uint16_t* dst = (n < kHeadDim ? k_cache : v_cache) + (size_t)bq * kv_stride +
                    (size_t)p * kHeadDim + (n & (kHeadDim - 1));
    *dst = f32_to_bf16_rne(sum);
  }
}

}  // namespace

hipError_t launch_bridge_decode(const uint16_t* h, int64_t ldh, const uint16_t* w_packed,
                                int rows, int d_model, const int32_t* pos, uint16_t* k_cache,
                                uint16_t* v_cache, int64_t kv_stride, int cap, hipStream_t st) {
  const dim3 grid(2 * kHeadDim / 32, (rows + 31) / 32);
  bridge_decode<<<grid, 64 * kBdWaves, 0, st>>>(h, ldh, w_packed, rows, d_model, pos, k_cache,
                                                v_cache, kv_stride, cap);
  return hipGetLastError();
}

}  // namespace hs2
