// Device helpers shared by the decode scoring kernels (bf16 and E4M3 K on
// v_mfma_f32_32x32x16_bf16).
#pragma once

#include "hs2_internal.h"

namespace hs2 {
namespace score {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Merge two (max, sum) pairs of base-2 softmax statistics.
__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both empty
  l = l * fast_exp2(m - mn) + l2 * fast_exp2(m2 - mn);
  m = mn;
}

// Registers of raw K per lane and 32-key block: 128 B of a bf16 row, 64 B of
// an E4M3 row.
template <bool kFp8>
constexpr int k_regs() {
  return kFp8 ? 4 : 8;
}

// Query rows as the MFMA operand of steps 0..7 (dims as step_dim gives).
template <bool kFp8>
__device__ __forceinline__ void load_q_bf16(const uint16_t* qb, int H, int r32, int hh,
                                            bf16x8_t (&qreg)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r32 < H) v = *reinterpret_cast<const u32x4*>(qb + r32 * kHeadDim + step_dim<kFp8>(i, hh));
    qreg[i] = as_bf16x8(v);
  }
}

// Lane half hh's share of key row `row` (kb: the sequence's cache, bytes):
// 16-byte pieces 2i + hh of the row.
template <bool kFp8>
__device__ __forceinline__ void load_k_block(const char* kb, int row, int hh,
                                             u32x4 (&kr)[k_regs<kFp8>()]) {
  const u32x4* kp =
      reinterpret_cast<const u32x4*>(kb + (size_t)row * kHeadDim * kv_elem_bytes<kFp8>()) + hh;
#pragma unroll
  for (int i = 0; i < k_regs<kFp8>(); ++i) kr[i] = kp[2 * i];
}

// The K operand of MFMA step e (compile-time after unrolling).
template <bool kFp8>
__device__ __forceinline__ bf16x8_t k_operand(const u32x4 (&kr)[k_regs<kFp8>()], int e) {
  if constexpr (kFp8)
    return as_bf16x8(e4m3x8_to_bf16x8(kr[e >> 1][2 * (e & 1)], kr[e >> 1][2 * (e & 1) + 1]));
  else
    return as_bf16x8(kr[e]);
}

}  // namespace score
}  // namespace hs2
