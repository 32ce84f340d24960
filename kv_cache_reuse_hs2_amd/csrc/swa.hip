// Sliding-window attention of the self-decoder's SWA layers.
//
// Prefill runs only the self-decoder, whose layers mix full attention with
// sliding-window attention ("HySparse2: How Xiaomi Split the Transformer to
// Fix Agent Prefill Costs", section "The Self-Decoder and Cross-Decoder
// Split").  A query at position P attends to the keys [max(0, P - W + 1), P]
// of one shared K/V head:
//   o_h = sum_j softmax(sm_scale * q_h . k_j) v_j.
//
// One workgroup takes 8 consecutive queries of a sequence (one per wave) and
// streams the union of their windows (W + 7 keys) through LDS in tiles of 64
// keys, K rows as they are (272-byte pitch, conflict-free operand reads) and
// V transposed.  Each wave runs a single-pass online softmax over 32-key
// chunks: QK^T is eight v_mfma_f32_32x32x16_bf16 with K as the A operand, so
// a lane holds one head over 16 keys; O is accumulated transposed,
// O^T += V^T P^T, so the lane that holds a head's running max also holds that
// head's 128 output columns (four 32x32 tiles) and the rescaling by
// 2^(m_old - m_new) needs no data movement.  The probabilities enter the P.V
// MFMAs as bf16 high and low parts (about fp32 accuracy), in the key order
// the QK^T result holds them, and the V^T operand is read in that same order.
#include "hs2_internal.h"

namespace hs2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kSwaWaves = 8;                // queries per workgroup, one per wave
constexpr int kSwaTile = 64;                // band keys per LDS tile
constexpr int kKPitch = kHeadDim * 2 + 16;  // bytes per staged K row
constexpr int kVtPitch = kSwaTile + 8;      // bf16 per transposed V row

struct SwaLds {
  uint8_t k[kSwaTile * kKPitch];
  uint16_t vt[kHeadDim][kVtPitch];
};

__global__ __launch_bounds__(64 * kSwaWaves) void swa_fwd_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t kv_stride, const int32_t* __restrict__ ctx_len,
    int cap, int n_q, int H, int window, float c2, float* __restrict__ o,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) SwaLds L;
  const int b = blockIdx.y, i0 = blockIdx.x * kSwaWaves;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  const int N = clamp_ctx(ctx_len, b, cap);
  const int i = i0 + wave;  // this wave's query
  const int P = N - n_q + i;
  const bool live = i < n_q && P >= 0;
  const int qlo = max(0, P - window + 1);  // this query's window [qlo, P]
  // The workgroup's band: the union of its queries' windows.
  const int p_first = N - n_q + i0, p_last = N - n_q + min(i0 + kSwaWaves, n_q) - 1;
  const int lo = max(0, p_first - window + 1);
  const int nb = p_last >= 0 ? p_last - lo + 1 : 0;

  bf16x8_t qr[8];
  {
    const uint16_t* qrow = q + ((size_t)b * n_q + min(i, n_q - 1)) * H * kHeadDim;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (live && r32 < H)
        x = *reinterpret_cast<const u32x4*>(qrow + r32 * kHeadDim + step_dim<false>(e, hh));
      qr[e] = as_bf16x8(x);
    }
  }
  const uint16_t* kb = k + (size_t)b * kv_stride;
  const uint16_t* vb = v + (size_t)b * kv_stride;

  float m_run = -INFINITY, l_run = 0.f;  // lane: head r32 (l_run over this half's keys)
  f32x16_t acc_o[4] = {{}, {}, {}, {}};  // O^T tiles: dims 32t + 8(r/4) + 4hh + r%4, head r32
  for (int t0 = 0; t0 < nb; t0 += kSwaTile) {
    __syncthreads();  // the previous tile is no longer read
    for (int e = threadIdx.x; e < kSwaTile * 16; e += blockDim.x) {
      const int r = e >> 4, c = e & 15;
      const size_t row = (size_t)min(lo + t0 + r, p_last) * kHeadDim + 8 * c;
      const u32x4 kx = *reinterpret_cast<const u32x4*>(kb + row);
      const u32x4 vx = *reinterpret_cast<const u32x4*>(vb + row);
      *reinterpret_cast<u32x4*>(L.k + r * kKPitch + 16 * c) = kx;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        L.vt[8 * c + 2 * u][r] = (uint16_t)(vx[u] & 0xFFFFu);
        L.vt[8 * c + 2 * u + 1][r] = (uint16_t)(vx[u] >> 16);
      }
    }
    __syncthreads();
    const int kt = min(kSwaTile, nb - t0);
    for (int c0 = 0; c0 < kt; c0 += 32) {
      const int a0 = lo + t0 + c0;  // key index of the chunk's first row
      if (!live || a0 > P || a0 + 31 < qlo) continue;  // chunk outside this window
      f32x16_t s = {};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bf16x8_t kop = as_bf16x8(*reinterpret_cast<const u32x4*>(
            L.k + (c0 + r32) * kKPitch + 32 * e + 16 * hh));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qr[e], s, 0, 0, 0);
      }
      // s[r]: head r32, key a0 + 8(r/4) + 4hh + r%4.
      float x[16];
      float bm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r >> 2) + 4 * hh + (r & 3);
        const int a = a0 + kk;
        x[r] = (c0 + kk < kt && a >= qlo && a <= P) ? s[r] * c2 : -INFINITY;
        bm = fmaxf(bm, x[r]);
      }
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float m_new = fmaxf(m_run, bm);
      const float mref = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - mref);
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = fast_exp2(x[r] - mref);
        ps += x[r];
      }
      l_run = l_run * alpha + ps;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[t][r] *= alpha;
      // O^T += V^T P^T over the chunk's two 16-key steps; step s takes the
      // keys of registers 8s..8s+7: {16s + 4hh + 0..3, 16s + 8 + 4hh + 0..3}.
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        u32x4 phi, plo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = x[8 * st + 2 * j], p1 = x[8 * st + 2 * j + 1];
          const uint16_t h0 = f32_to_bf16_rne(p0), h1 = f32_to_bf16_rne(p1);
          const uint16_t l0 = f32_to_bf16_rne(p0 - bf16_to_f32(h0));
          const uint16_t l1 = f32_to_bf16_rne(p1 - bf16_to_f32(h1));
          phi[j] = (uint32_t)h0 | ((uint32_t)h1 << 16);
          plo[j] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint16_t* vrow = &L.vt[32 * t + r32][c0];
          const uint2 lo4 = *reinterpret_cast<const uint2*>(vrow + 16 * st + 4 * hh);
          const uint2 hi4 = *reinterpret_cast<const uint2*>(vrow + 16 * st + 8 + 4 * hh);
          const u32x4 av = {lo4.x, lo4.y, hi4.x, hi4.y};
          acc_o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(phi),
                                                             acc_o[t], 0, 0, 0);
          acc_o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(plo),
                                                             acc_o[t], 0, 0, 0);
        }
      }
    }
  }
  if (i >= n_q) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (r32 >= H) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  float* orow = o + (((size_t)b * n_q + i) * H + r32) * kHeadDim;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 val = {acc_o[t][4 * g] * inv, acc_o[t][4 * g + 1] * inv,
                         acc_o[t][4 * g + 2] * inv, acc_o[t][4 * g + 3] * inv};
      *reinterpret_cast<f32x4*>(orow + 32 * t + 8 * g + 4 * hh) = val;
    }
  if (lse != nullptr && hh == 0)
    lse[((size_t)b * n_q + i) * H + r32] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_swa(const hs2_attn_desc& d, const void* q, const void* k, const void* v,
                      int64_t kv_stride, const int32_t* ctx_len, int cap, float* o, float* lse,
                      hipStream_t st) {
  const dim3 grid((d.n_q + kSwaWaves - 1) / kSwaWaves, d.batch);
  swa_fwd_bf16<<<grid, 64 * kSwaWaves, 0, st>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), kv_stride, ctx_len, cap, d.n_q, d.n_heads, d.window,
      d.sm_scale * kLog2e, o, lse);
  return hipGetLastError();
}

}  // namespace hs2
