// Full-attention scoring for a decode step (one query per sequence).
//
// The full layer of a hybrid block attends over the whole context and, from
// that attention, yields the token selection the sparse layers reuse
// ("HySparse2: How Xiaomi Split the Transformer to Fix Agent Prefill Costs",
// section "KV Reuse and Token-Level Sparse Selection").  The per-key
// importance is the softmax probability summed over all query heads:
//   I[j] = sum_h 2^(x_hj - L_h),  x_hj = (sm_scale*log2 e) * q_h.k_j,
//   L_h  = log2 sum_j 2^(x_hj)    (base-2 log-sum-exp of head h).
// L_h needs every key before any I[j] exists, so the K cache is streamed
// twice, with the kernel boundary as the only synchronisation (on this chip
// a release/acquire between workgroups writes back the L2 and costs more
// than the second read):
//   pass 1: per 4,096-key chunk, per-head (max, sum);
//   pass 2: per 4,096-key chunk, each workgroup first folds the chunk
//           statistics of its sequence into L_h (a few KiB from L2), then
//           recomputes the logits and writes I; optionally it also adds the
//           chunk's histogram of score bits (pool keys only) to the
//           selector's per-sequence histogram.  Pass 2 walks the chunks in
//           the reverse order of pass 1, so its first reads hit what the
//           memory-side cache still holds.
//
// bf16 path: one wave computes a 32-key x 32-head logit tile with eight
// v_mfma_f32_32x32x16_bf16 (K = 128 = 8 x 16).  Each lane loads 16 B of a key
// row per MFMA step straight from HBM (lane%32 = key, lane/32 = which 8 dims
// of the 16-dim step) and the next block is prefetched while the current one
// is in the MFMA.  Pass 1 takes K as the A operand so that a lane holds one
// head over 16 keys (per-head max/sum are in-lane); pass 2 takes K as the B
// operand so that a lane holds one key over 16 heads (the head sum is
// in-lane plus one cross-half add).
//
// E4M3 path: the same kernels read 64 B of a key row per lane and widen the
// bytes to bf16 in registers (exact), so the MFMA work is unchanged and the
// HBM stream halves.  The cache scale multiplies the logit scale:
// sm_scale * q.(s k) = (sm_scale * s) * q.k.
//
// fp32 path: a VALU dot-product kernel, one key per thread, with a separate
// reduction kernel.
#include "score_common.h"

namespace hs2 {
namespace {

using namespace score;

constexpr int kP1Waves = 8;
constexpr int kP2Waves = 8;

// Pass 1, bf16 or E4M3 K: per (sequence, chunk, head) base-2 (max, sum).
// Chunks at or beyond the context write neutral statistics.  The workgroup of
// chunk 0 also clears the sequence's selector histogram when one is built.
template <bool kFp8>
__global__ __launch_bounds__(64 * kP1Waves) void score_p1_bf16(
    const uint16_t* __restrict__ q, const void* __restrict__ k, int64_t kv_stride,
    const int32_t* __restrict__ ctx_len, int cap, int H, float c2, float2* __restrict__ stats,
    int nchunks, uint32_t* __restrict__ hist) {
  const int b = blockIdx.y, c = blockIdx.x;
  const int N = clamp_ctx(ctx_len, b, cap);
  const int j_begin = c * kP1Chunk;
  float2* st = stats + ((size_t)b * nchunks + c) * kMaxHeads;
  if (hist != nullptr && c == 0)
    for (int i = threadIdx.x; i < kHistRow; i += blockDim.x) hist[(size_t)b * kHistRow + i] = 0u;
  if (j_begin >= N) {
    if (threadIdx.x < kMaxHeads) st[threadIdx.x] = make_float2(-INFINITY, 0.f);
    return;
  }
  const int j_end = min(N, j_begin + kP1Chunk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;

  bf16x8_t qreg[8];
  load_q_bf16<kFp8>(q + (size_t)b * H * kHeadDim, H, r32, hh, qreg);
  const char* kb = static_cast<const char*>(k) + (size_t)b * kv_stride * kv_elem_bytes<kFp8>();

  float m_run = -INFINITY, l_run = 0.f;
  int j0 = j_begin + 32 * wave;
  u32x4 ka[k_regs<kFp8>()], kn[k_regs<kFp8>()];
  if (j0 < j_end) load_k_block<kFp8>(kb, min(j0 + r32, N - 1), hh, ka);
  auto block = [&](const u32x4 (&kc)[k_regs<kFp8>()], const int jb) {
    f32x16_t acc = {};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand<kFp8>(kc, i), qreg[i], acc, 0, 0, 0);
    // acc[r] = logit of key jb + 8*(r/4) + 4*hh + r%4 for head r32.
    float x[16];
    float bm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = jb + 8 * (r >> 2) + 4 * hh + (r & 3);
      x[r] = (j < j_end) ? acc[r] * c2 : -INFINITY;
      bm = fmaxf(bm, x[r]);
    }
    const float m_new = fmaxf(m_run, bm);
    const float mref = (m_new == -INFINITY) ? 0.f : m_new;
    float s = l_run * fast_exp2(m_run - mref);
#pragma unroll
    for (int r = 0; r < 16; ++r) s += fast_exp2(x[r] - mref);
    l_run = s;
    m_run = m_new;
  };
  // Two register sets used in turn, so the next block's loads stay in flight
  // while the current block is computed.  The loads are unconditional (past
  // the end they repeat the current block, which the cache still holds): a
  // load under a branch, or a copy between the sets, makes the compiler wait
  // for every load in flight before the next MFMA.
  constexpr int kStep = 32 * kP1Waves;
  while (j0 < j_end) {
    const int j1 = j0 + kStep;
    load_k_block<kFp8>(kb, min((j1 < j_end ? j1 : j0) + r32, N - 1), hh, kn);
    __builtin_amdgcn_sched_barrier(0);  // issue the loads before the wait below
    block(ka, j0);
    if (j1 >= j_end) break;
    const int j2 = j1 + kStep;
    load_k_block<kFp8>(kb, min((j2 < j_end ? j2 : j1) + r32, N - 1), hh, ka);
    __builtin_amdgcn_sched_barrier(0);
    block(kn, j1);
    j0 = j2;
  }
  // Lanes r32 and r32+32 hold the same head over different keys.
  merge_ml(m_run, l_run, __shfl_xor(m_run, 32), __shfl_xor(l_run, 32));
  __shared__ float2 part[kP1Waves][32];
  if (hh == 0) part[wave][r32] = make_float2(m_run, l_run);
  __syncthreads();
  if (threadIdx.x < 32) {
    float m = part[0][threadIdx.x].x, l = part[0][threadIdx.x].y;
#pragma unroll
    for (int w = 1; w < kP1Waves; ++w) merge_ml(m, l, part[w][threadIdx.x].x, part[w][threadIdx.x].y);
    st[threadIdx.x] = make_float2(m, l);
  }
}

// Pass 2, bf16 or E4M3 K: fold the statistics into L_h, then
// I[j] = sum_h 2^(x_hj - L_h).  kHist: also count the pool scores into the
// selector's first histogram.
template <bool kFp8, bool kHist>
__global__ __launch_bounds__(64 * kP2Waves) void score_p2_bf16(
    const uint16_t* __restrict__ q, const void* __restrict__ k, int64_t kv_stride,
    const int32_t* __restrict__ ctx_len, int cap, int H, float c2,
    const float2* __restrict__ stats, int nchunks1, float* __restrict__ scores,
    int64_t score_stride, float* __restrict__ lse_out, uint32_t* __restrict__ hist,
    int window) {
  const int b = gridDim.y - 1 - blockIdx.y;
  const int c = gridDim.x - 1 - blockIdx.x;
  const int N = clamp_ctx(ctx_len, b, cap);
  const int j_begin = c * kP2Chunk;
  if (j_begin >= N) {
    if (lse_out != nullptr && c == 0 && threadIdx.x < H) lse_out[b * H + threadIdx.x] = -INFINITY;
    return;
  }
  const int j_end = min(N, j_begin + kP2Chunk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  const char* kb = static_cast<const char*>(k) + (size_t)b * kv_stride * kv_elem_bytes<kFp8>();

  // Start the K stream before folding the statistics.
  int j0 = j_begin + 32 * wave;
  u32x4 ka[k_regs<kFp8>()], kn[k_regs<kFp8>()];
  if (j0 < j_end) load_k_block<kFp8>(kb, min(j0 + r32, N - 1), hh, ka);
  bf16x8_t qreg[8];
  load_q_bf16<kFp8>(q + (size_t)b * H * kHeadDim, H, r32, hh, qreg);

  constexpr int kParts = kP2Waves * 2;  // 32-thread groups folding the statistics
  __shared__ float2 red[kParts][32];
  __shared__ float s_L[32];
  __shared__ uint32_t s_hist[kHist ? kSelBins : 1];
  {
    const int h = threadIdx.x & 31, part = threadIdx.x >> 5;
    const int nc = (N + kP1Chunk - 1) / kP1Chunk;
    const float2* sb = stats + (size_t)b * nchunks1 * kMaxHeads;
    float m = -INFINITY, l = 0.f;
    for (int cc = part; cc < nc; cc += kParts) {
      const float2 v = sb[(size_t)cc * kMaxHeads + h];
      merge_ml(m, l, v.x, v.y);
    }
    red[part][h] = make_float2(m, l);
    if (kHist)
      for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) s_hist[i] = 0u;
    __syncthreads();
    if (threadIdx.x < 32) {
      m = red[0][h].x;
      l = red[0][h].y;
#pragma unroll
      for (int p = 1; p < kParts; ++p) merge_ml(m, l, red[p][h].x, red[p][h].y);
      const float L = (l > 0.f) ? m + log2f(l) : -INFINITY;
      s_L[h] = (h < H) ? L : INFINITY;  // padded heads contribute 2^-inf = 0
      if (lse_out != nullptr && c == 0 && h < H) lse_out[b * H + h] = L * 0.69314718055994531f;
    }
    __syncthreads();
  }
  float L[16];  // lane holds heads 8*(r/4) + 4*hh + r%4
#pragma unroll
  for (int r = 0; r < 16; ++r) L[r] = s_L[8 * (r >> 2) + 4 * hh + (r & 3)];
  float* out = scores + (size_t)b * score_stride;
  const int pe = N - window;  // decode pool end (keys below it are histogrammed)

  auto block = [&](const u32x4 (&kc)[k_regs<kFp8>()], const int jb) {
    f32x16_t acc = {};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qreg[i], k_operand<kFp8>(kc, i), acc, 0, 0, 0);
    // acc[r] = logit of head 8*(r/4) + 4*hh + r%4 for key jb + r32.
    float imp = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) imp += fast_exp2(acc[r] * c2 - L[r]);
    imp += __shfl_xor(imp, 32);
    const int j = jb + r32;
    if (hh == 0 && j < j_end) {
      out[j] = imp;
      if (kHist && j < pe) atomicAdd(&s_hist[order_key(imp) >> 20], 1u);
    }
  };
  // Two register sets used in turn, with unconditional loads, as in pass 1.
  constexpr int kStep = 32 * kP2Waves;
  while (j0 < j_end) {
    const int j1 = j0 + kStep;
    load_k_block<kFp8>(kb, min((j1 < j_end ? j1 : j0) + r32, N - 1), hh, kn);
    __builtin_amdgcn_sched_barrier(0);  // issue the loads before the wait below
    block(ka, j0);
    if (j1 >= j_end) break;
    const int j2 = j1 + kStep;
    load_k_block<kFp8>(kb, min((j2 < j_end ? j2 : j1) + r32, N - 1), hh, ka);
    __builtin_amdgcn_sched_barrier(0);
    block(kn, j1);
    j0 = j2;
  }
  if (kHist) {
    __syncthreads();
    uint32_t* gh = hist + (size_t)b * kHistRow;
    for (int i = threadIdx.x; i < kSelBins; i += blockDim.x)
      if (s_hist[i] != 0u) atomicAdd(&gh[i], s_hist[i]);
  }
}

// ---------------------------------------------------------------------------
// Pass 2 with the full layer's own output: besides I[j], each workgroup adds
// p_hj v_j over its 4,096 keys into a partial O, and full_out_combine sums the
// partials of a sequence in chunk order (p_hj = 2^(x_hj - L_h) is already
// normalised, so partials simply add).  Here K is the A operand, so a lane
// holds one head over 16 keys: O is accumulated transposed, O^T += V^T P^T,
// with P as bf16 high and low parts and V transposed through the wave's LDS
// tile; the importance (a sum over heads, i.e. over lanes) goes through a
// 32 x 32 transpose in LDS.
constexpr int kFullVt = 40;  // bf16 per transposed V row (32 keys + pad)

struct FullLds {
  float2 red[kP2Waves * 2][32];
  float s_L[32];
  union {
    struct {
      uint16_t vt[kP2Waves][kHeadDim][kFullVt];
      float pt[kP2Waves][32][33];
    } loop;
    float merge[kP2Waves / 2][32][kHeadDim + 4];
  } u;
};

// V rows are read like K rows (load_k_block: each load instruction covers 32
// B of 32 rows); group e of the lane's values, widened to bf16, holds dims
// step_dim(e, hh) .. +8.
template <bool kFp8>
__device__ __forceinline__ u32x4 v_dims8(const u32x4 (&vr)[k_regs<kFp8>()], int e) {
  if constexpr (kFp8)
    return e4m3x8_to_bf16x8(vr[e >> 1][2 * (e & 1)], vr[e >> 1][2 * (e & 1) + 1]);
  else
    return vr[e];
}

template <bool kFp8>
__global__ __launch_bounds__(64 * kP2Waves) void score_p2_full(
    const uint16_t* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    int64_t kv_stride, const int32_t* __restrict__ ctx_len, int cap, int H, float c2,
    const float2* __restrict__ stats, int nchunks1, float* __restrict__ scores,
    int64_t score_stride, float* __restrict__ lse_out, float* __restrict__ o_part,
    int nchunks2) {
  __shared__ __attribute__((aligned(16))) FullLds S;
  const int b = gridDim.y - 1 - blockIdx.y;
  const int c = gridDim.x - 1 - blockIdx.x;
  const int N = clamp_ctx(ctx_len, b, cap);
  const int j_begin = c * kP2Chunk;
  if (j_begin >= N) {
    if (lse_out != nullptr && c == 0 && threadIdx.x < H) lse_out[b * H + threadIdx.x] = -INFINITY;
    return;
  }
  const int j_end = min(N, j_begin + kP2Chunk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  const size_t seq = (size_t)b * kv_stride * kv_elem_bytes<kFp8>();
  const char* kb = static_cast<const char*>(k) + seq;
  const char* vb = static_cast<const char*>(v) + seq;

  int j0 = j_begin + 32 * wave;
  u32x4 kr[k_regs<kFp8>()], vr[k_regs<kFp8>()];
  if (j0 < j_end) {
    load_k_block<kFp8>(kb, min(j0 + r32, N - 1), hh, kr);
    load_k_block<kFp8>(vb, min(j0 + r32, N - 1), hh, vr);
  }
  bf16x8_t qreg[8];
  load_q_bf16<kFp8>(q + (size_t)b * H * kHeadDim, H, r32, hh, qreg);
  {
    constexpr int kParts = kP2Waves * 2;
    const int h = threadIdx.x & 31, part = threadIdx.x >> 5;
    const int nc = (N + kP1Chunk - 1) / kP1Chunk;
    const float2* sb = stats + (size_t)b * nchunks1 * kMaxHeads;
    float m = -INFINITY, l = 0.f;
    for (int cc = part; cc < nc; cc += kParts) {
      const float2 x = sb[(size_t)cc * kMaxHeads + h];
      merge_ml(m, l, x.x, x.y);
    }
    S.red[part][h] = make_float2(m, l);
    __syncthreads();
    if (threadIdx.x < 32) {
      m = S.red[0][h].x;
      l = S.red[0][h].y;
#pragma unroll
      for (int p = 1; p < kParts; ++p) merge_ml(m, l, S.red[p][h].x, S.red[p][h].y);
      const float L = (l > 0.f) ? m + log2f(l) : -INFINITY;
      S.s_L[h] = (h < H) ? L : INFINITY;  // padded heads get p = 0
      if (lse_out != nullptr && c == 0 && h < H) lse_out[b * H + h] = L * 0.69314718055994531f;
    }
    __syncthreads();
  }
  const float Lh = S.s_L[r32];
  float* out = scores + (size_t)b * score_stride;
  f32x16_t o[4] = {{}, {}, {}, {}};  // O^T: dims 32t + 8(r/4) + 4hh + r%4, head r32
  float (*pt)[33] = S.u.loop.pt[wave];
  uint16_t (*vt)[kFullVt] = S.u.loop.vt[wave];
  // Each wave's next block is loaded into the same registers as soon as the
  // QK^T MFMAs and the V transpose have consumed them, so the loads are in
  // flight during the rest of the block's work.
  while (j0 < j_end) {
    const int jn = j0 + 32 * kP2Waves;
    f32x16_t acc = {};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand<kFp8>(kr, i), qreg[i], acc, 0, 0,
                                                    0);
    // V transposed: vt[d][key r32], d = step_dim(e, hh) + 2j (+ 1).
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const u32x4 x = v_dims8<kFp8>(vr, e);
      const int d0 = step_dim<kFp8>(e, hh);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vt[d0 + 2 * j][r32] = (uint16_t)(x[j] & 0xFFFFu);
        vt[d0 + 2 * j + 1][r32] = (uint16_t)(x[j] >> 16);
      }
    }
    if (jn < j_end) {
      load_k_block<kFp8>(kb, min(jn + r32, N - 1), hh, kr);
      load_k_block<kFp8>(vb, min(jn + r32, N - 1), hh, vr);
    }
    // acc[r]: head r32, key j0 + 8(r/4) + 4hh + r%4.
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = 8 * (r >> 2) + 4 * hh + (r & 3);
      p[r] = (j0 + kk < j_end) ? fast_exp2(acc[r] * c2 - Lh) : 0.f;
      pt[r32][kk] = p[r];
    }
    wave_lds_sync();  // the two tiles are this wave's alone
    // I[j] = sum over heads: lane (key r32, half hh) adds heads 16hh .. 16hh + 15.
    float imp = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) imp += pt[16 * hh + i][r32];
    imp += __shfl_xor(imp, 32);
    if (hh == 0 && j0 + r32 < j_end) out[j0 + r32] = imp;
    // O^T += V^T P^T; step s takes the keys of registers 8s..8s+7.
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      u32x4 phi, plo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = p[8 * sp + 2 * j], p1 = p[8 * sp + 2 * j + 1];
        const uint16_t h0 = f32_to_bf16_rne(p0), h1 = f32_to_bf16_rne(p1);
        const uint16_t l0 = f32_to_bf16_rne(p0 - bf16_to_f32(h0));
        const uint16_t l1 = f32_to_bf16_rne(p1 - bf16_to_f32(h1));
        phi[j] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        plo[j] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint16_t* vrow = &vt[32 * t + r32][0];
        const uint2 lo4 = *reinterpret_cast<const uint2*>(vrow + 16 * sp + 4 * hh);
        const uint2 hi4 = *reinterpret_cast<const uint2*>(vrow + 16 * sp + 8 + 4 * hh);
        const u32x4 av = {lo4.x, lo4.y, hi4.x, hi4.y};
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(phi), o[t], 0,
                                                       0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(plo), o[t], 0,
                                                       0, 0);
      }
    }
    wave_lds_sync();  // reads above before the next block's writes
    j0 = jn;
  }
  // The 8 waves' partials, added in a fixed tree (4 + 4, 2 + 2, 1 + 1).
  __syncthreads();  // the loop's LDS tiles are reused below
#pragma unroll
  for (int half = kP2Waves / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          S.u.merge[wave - half][r32][32 * t + 8 * (r >> 2) + 4 * hh + (r & 3)] = o[t][r];
    }
    __syncthreads();
    if (wave < half) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          o[t][r] += S.u.merge[wave][r32][32 * t + 8 * (r >> 2) + 4 * hh + (r & 3)];
    }
    __syncthreads();
  }
  if (wave == 0 && r32 < H) {
    float* dst = o_part + (((size_t)b * nchunks2 + c) * kMaxHeads + r32) * kHeadDim;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = {o[t][4 * g], o[t][4 * g + 1], o[t][4 * g + 2], o[t][4 * g + 3]};
        *reinterpret_cast<f32x4*>(dst + 32 * t + 8 * g + 4 * hh) = x;
      }
  }
}

// o_full[b][h][:] = v_scale * sum of the sequence's chunk partials: thread
// group g (of 16) adds chunks g, g + 16, ... in order, then group 0 adds the
// 16 group sums in order.  Four dims per thread.
constexpr int kCombGroups = 16;

__global__ __launch_bounds__(32 * kCombGroups) void full_out_combine(
    const float* __restrict__ o_part, int nchunks2, const int32_t* __restrict__ ctx_len, int cap,
    int H, float v_scale, float* __restrict__ o_full) {
  __shared__ f32x4 red[kCombGroups][32];
  const int h = blockIdx.x, b = blockIdx.y;
  const int d4 = threadIdx.x & 31, g = threadIdx.x >> 5;
  const int N = clamp_ctx(ctx_len, b, cap);
  const int nc = (N + kP2Chunk - 1) / kP2Chunk;
  const f32x4* src =
      reinterpret_cast<const f32x4*>(o_part + ((size_t)b * nchunks2 * kMaxHeads + h) * kHeadDim) +
      d4;
  constexpr size_t kChunkStride = kMaxHeads * kHeadDim / 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c = g; c < nc; c += kCombGroups) acc += src[(size_t)c * kChunkStride];
  red[g][d4] = acc;
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int i = 1; i < kCombGroups; ++i) acc += red[i][d4];
    *reinterpret_cast<f32x4*>(o_full + ((size_t)b * H + h) * kHeadDim + 4 * d4) = acc * v_scale;
  }
}

// L_h = m + log2(l) of sequence b over its nc chunk statistics, for every
// head slot h < 32: eight interleaved parts (part p merges chunks p, p + 8,
// ...) are merged in part order.  Any block size; threads t < 32 return L of
// head t (others 0).  red: LDS [8][32].
__device__ float reduce_chunk_stats(const float2* __restrict__ stats_b, int nc,
                                    float2 (*red)[32]) {
  for (int i = threadIdx.x; i < 8 * 32; i += blockDim.x) {
    const int h = i & 31, part = i >> 5;
    float m = -INFINITY, l = 0.f;
    for (int c = part; c < nc; c += 8) {
      const float2 s = stats_b[(size_t)c * kMaxHeads + h];
      merge_ml(m, l, s.x, s.y);
    }
    red[part][h] = make_float2(m, l);
  }
  __syncthreads();
  float L = 0.f;
  if (threadIdx.x < 32) {
    const int h = threadIdx.x;
    float m = red[0][h].x, l = red[0][h].y;
    for (int p = 1; p < 8; ++p) merge_ml(m, l, red[p][h].x, red[p][h].y);
    L = (l > 0.f) ? m + log2f(l) : -INFINITY;
  }
  return L;
}

// fp32 VALU kernel: MODE 0 writes per-chunk statistics (and its chunk-0
// workgroup clears the sequence's selector histograms, when given), MODE 1
// importance: each workgroup first merges the sequence's chunk statistics
// into L_h itself (as score_reduce_f32 does, the same bits), so no launch
// sits between the passes; the chunk-0 workgroup also writes the full
// layer's lse.  A workgroup takes 64 keys (one per lane) and kHB >= H heads
// (8, 16 or 32; the rows past H are zero), kF32Heads heads per wave, so that
// a thread runs kF32Heads fma chains rather than all kHB.  Each logit is one
// fma chain over the 128 dims in order, the same chain score_full_f32 runs;
// MODE 1 adds a key's head terms in head order in one thread (through LDS),
// so both write the same importance bits.
constexpr int kF32Heads = 4;

template <int MODE, int kHB>
__global__ __launch_bounds__(kF32Chunk * kHB / kF32Heads) void score_f32(
    const float* __restrict__ q, const float* __restrict__ k, int64_t kv_stride,
    const int32_t* __restrict__ ctx_len, int cap, int H, float c2,
    float2* __restrict__ stats, int nchunks, float* __restrict__ lse_out,
    float* __restrict__ scores, int64_t score_stride, uint32_t* __restrict__ hist, int window) {
  static_assert(kF32Chunk == 64 && kHB % kF32Heads == 0, "a key per lane, whole head groups");
  const int b = blockIdx.y;
  const int c = (MODE == 1) ? (gridDim.x - 1 - blockIdx.x) : blockIdx.x;
  const int N = clamp_ctx(ctx_len, b, cap);
  if (MODE == 0 && hist != nullptr && c == 0)
    for (int i = threadIdx.x; i < kHistRow; i += blockDim.x) hist[(size_t)b * kHistRow + i] = 0u;
  const int j_begin = c * kF32Chunk;
  if (j_begin >= N) {  // workgroup-uniform
    // An empty sequence: no statistics to merge, lse -inf.
    if (MODE == 1 && N == 0 && c == 0 && lse_out != nullptr && threadIdx.x < H)
      lse_out[b * H + threadIdx.x] = -INFINITY;
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h0 = kF32Heads * wave;  // this wave's heads
  __shared__ float4 qs[kHB][kHeadDim / 4];
  __shared__ float4 ks[kF32Chunk][kHeadDim / 4 + 1];  // padded: a lane per row
  __shared__ float terms[kF32Chunk][kHB + 1];         // MODE 1: a key's head terms
  __shared__ float2 red[8][32];                        // MODE 1: statistics merge
  __shared__ float s_L[32];                            // MODE 1: L_h
  // Q and the chunk's K rows through LDS, every load of a thread issued at
  // once (one round trip; K 512 contiguous bytes per 32 threads), then the
  // statistics merge, whose loads overlap those.
  {
    constexpr int kThreads = kF32Chunk * kHB / kF32Heads;
    constexpr int kPer = kF32Chunk * (kHeadDim / 4) / kThreads;
    constexpr int kPerQ = kHB * (kHeadDim / 4) / kThreads;
    const float* kb = k + (size_t)b * kv_stride;
    const float* qb = q + (size_t)b * H * kHeadDim;
    float4 x[kPer], y[kPerQ];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = threadIdx.x + i * kThreads, r = e / (kHeadDim / 4), d4 = e % (kHeadDim / 4);
      x[i] = reinterpret_cast<const float4*>(kb + (size_t)min(j_begin + r, N - 1) * kHeadDim)[d4];
    }
#pragma unroll
    for (int i = 0; i < kPerQ; ++i) {
      const int e = threadIdx.x + i * kThreads, h = e / (kHeadDim / 4), d4 = e % (kHeadDim / 4);
      y[i] = h < H ? reinterpret_cast<const float4*>(qb + h * kHeadDim)[d4]
                   : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (MODE == 1) {
      const float L = reduce_chunk_stats(stats + (size_t)b * nchunks * kMaxHeads,
                                         (N + kF32Chunk - 1) / kF32Chunk, red);
      if (threadIdx.x < 32) {
        const int h = threadIdx.x;
        s_L[h] = (h < H) ? L : INFINITY;  // padded heads: 2^-inf = 0
        if (lse_out != nullptr && c == 0 && h < H) lse_out[b * H + h] = L * 0.69314718055994531f;
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = threadIdx.x + i * kThreads;
      ks[e / (kHeadDim / 4)][e % (kHeadDim / 4)] = x[i];
    }
#pragma unroll
    for (int i = 0; i < kPerQ; ++i) {
      const int e = threadIdx.x + i * kThreads;
      qs[e / (kHeadDim / 4)][e % (kHeadDim / 4)] = y[i];
    }
  }
  __syncthreads();
  const int j = j_begin + lane;
  const bool valid = j < N;
  float acc[kF32Heads];
#pragma unroll
  for (int u = 0; u < kF32Heads; ++u) acc[u] = 0.f;
#pragma unroll 8
  for (int d4 = 0; d4 < kHeadDim / 4; ++d4) {
    const float4 kv = ks[lane][d4];
#pragma unroll
    for (int u = 0; u < kF32Heads; ++u) {
      const float4 qv = qs[h0 + u][d4];
      acc[u] = fmaf(qv.x, kv.x, acc[u]);
      acc[u] = fmaf(qv.y, kv.y, acc[u]);
      acc[u] = fmaf(qv.z, kv.z, acc[u]);
      acc[u] = fmaf(qv.w, kv.w, acc[u]);
    }
  }
  if (MODE == 1) {
#pragma unroll
    for (int u = 0; u < kF32Heads; ++u) {
      const int h = h0 + u;
      terms[lane][h] = h < H ? fast_exp2(acc[u] * c2 - s_L[h]) : 0.f;
    }
    __syncthreads();
    if (wave != 0 || !valid) return;
    float imp = 0.f;
#pragma unroll
    for (int h = 0; h < kHB; ++h)
      if (h < H) imp += terms[lane][h];
    scores[(size_t)b * score_stride + j] = imp;
    // The selector's first histogram (pool keys only; cleared by the
    // statistics pass).  The wave's keys are grouped by
    // bin first, one atomic per distinct bin: the scores crowd into few bins.
    if (hist != nullptr) {
      const uint32_t bin = order_key(imp) >> 20;
      bool todo = j < N - window;
      while (__ballot(todo) != 0ull) {  // wave-uniform
        if (todo) {
          const uint32_t lead = __builtin_amdgcn_readfirstlane(bin);
          const uint64_t same = __ballot(bin == lead);
          if (bin == lead) {
            todo = false;
            if (lane == __ffsll((unsigned long long)same) - 1)
              atomicAdd(&hist[(size_t)b * kHistRow + lead], (uint32_t)__popcll(same));
          }
        }
      }
    }
  } else {
    float2* st = stats + ((size_t)b * nchunks + c) * kMaxHeads;
#pragma unroll
    for (int u = 0; u < kF32Heads; ++u) {
      const float x = valid ? acc[u] * c2 : -INFINITY;
      float m = x;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      float s = fast_exp2(x - (m == -INFINITY ? 0.f : m));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
      if (lane == 0) st[h0 + u] = make_float2(m, s);
    }
    // Heads past the bucket: neutral statistics (never used for a real head).
    if (threadIdx.x < kMaxHeads - kHB) st[kHB + threadIdx.x] = make_float2(-INFINITY, 0.f);
  }
}

// The head bucket of H for score_f32.
template <int MODE>
void launch_score_f32(dim3 grid, hipStream_t st, const float* q, const float* k,
                      int64_t kv_stride, const int32_t* ctx_len, int cap, int H, float c2,
                      float2* stats, int nchunks, float* lse_out, float* scores,
                      int64_t score_stride, uint32_t* hist = nullptr, int window = 0) {
  constexpr int kW = kF32Chunk / kF32Heads;  // threads per head of the bucket
  if (H <= 8)
    score_f32<MODE, 8><<<grid, 8 * kW, 0, st>>>(q, k, kv_stride, ctx_len, cap, H, c2, stats,
                                               nchunks, lse_out, scores, score_stride, hist, window);
  else if (H <= 16)
    score_f32<MODE, 16><<<grid, 16 * kW, 0, st>>>(q, k, kv_stride, ctx_len, cap, H, c2, stats,
                                                 nchunks, lse_out, scores, score_stride,
                                                 hist, window);
  else
    score_f32<MODE, 32><<<grid, 32 * kW, 0, st>>>(q, k, kv_stride, ctx_len, cap, H, c2, stats,
                                                 nchunks, lse_out, scores, score_stride,
                                                 hist, window);
}

// fp32 path with the full layer's own output: workgroup (c, b) takes keys
// [4096c, 4096c + 4096) in sub-blocks of 256.  Per sub-block a thread owns
// one key: it computes the 32 logits as score_f32<1> does, writes I[j] (the
// same arithmetic, so the same bits) and puts p_hj in LDS; then a thread owns
// output dim t % 128 of heads 16(t / 128) .. + 15 and adds p_hj v_jd over
// the sub-block's keys in order.  The chunk's partial O goes to o_part[b][c]
// for full_out_combine, as in the MFMA paths.
__global__ __launch_bounds__(256) void score_full_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    int64_t kv_stride, const int32_t* __restrict__ ctx_len, int cap, int H, float c2,
    const float* __restrict__ lse2, float* __restrict__ scores, int64_t score_stride,
    float* __restrict__ o_part, int nchunks2) {
  const int b = blockIdx.y, c = blockIdx.x;
  const int N = clamp_ctx(ctx_len, b, cap);
  const int j_begin = c * kP2Chunk;
  if (j_begin >= N) return;
  const int j_end = min(N, j_begin + kP2Chunk);
  __shared__ float4 qs[kMaxHeads][kHeadDim / 4];
  __shared__ float ps[kMaxHeads][kF32Sub];
  const float* qb = q + (size_t)b * H * kHeadDim;
  for (int e = threadIdx.x; e < kMaxHeads * kHeadDim / 4; e += blockDim.x) {
    const int h = e / (kHeadDim / 4), d4 = e % (kHeadDim / 4);
    qs[h][d4] = h < H ? reinterpret_cast<const float4*>(qb + h * kHeadDim)[d4]
                      : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float* kb = k + (size_t)b * kv_stride;
  const float* vb = v + (size_t)b * kv_stride;
  const int d = threadIdx.x & (kHeadDim - 1), hg = threadIdx.x >> 7;
  float oacc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) oacc[i] = 0.f;
  for (int j0 = j_begin; j0 < j_end; j0 += kF32Sub) {
    __syncthreads();  // q staged; the previous sub-block's ps read
    const int j = j0 + threadIdx.x;
    const bool valid = j < j_end;
    const float4* kp = reinterpret_cast<const float4*>(kb + (size_t)min(j, N - 1) * kHeadDim);
    float acc[kMaxHeads];
#pragma unroll
    for (int h = 0; h < kMaxHeads; ++h) acc[h] = 0.f;
#pragma unroll 8
    for (int d4 = 0; d4 < kHeadDim / 4; ++d4) {
      const float4 kv = kp[d4];
#pragma unroll
      for (int h = 0; h < kMaxHeads; ++h) {
        const float4 qv = qs[h][d4];
        acc[h] = fmaf(qv.x, kv.x, acc[h]);
        acc[h] = fmaf(qv.y, kv.y, acc[h]);
        acc[h] = fmaf(qv.z, kv.z, acc[h]);
        acc[h] = fmaf(qv.w, kv.w, acc[h]);
      }
    }
    float imp = 0.f;
#pragma unroll
    for (int h = 0; h < kMaxHeads; ++h) {
      const float p = (valid && h < H) ? fast_exp2(acc[h] * c2 - lse2[b * kMaxHeads + h]) : 0.f;
      if (h < H) imp += p;
      ps[h][threadIdx.x] = p;
    }
    if (valid) scores[(size_t)b * score_stride + j] = imp;
    __syncthreads();
    const int nk = min(kF32Sub, j_end - j0);
    for (int jj = 0; jj < nk; ++jj) {
      const float x = vb[(size_t)(j0 + jj) * kHeadDim + d];
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[i] = fmaf(ps[16 * hg + i][jj], x, oacc[i]);
    }
  }
  float* dst = o_part + ((size_t)b * nchunks2 + c) * kMaxHeads * kHeadDim + d;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (16 * hg + i < H) dst[(size_t)(16 * hg + i) * kHeadDim] = oacc[i];
}

// fp32 path with the full layer's own output: per (sequence, head) L_h for
// score_full_f32 (and the full layer's lse); heads beyond H get +inf so that
// 2^(x - L) vanishes for them.  Also clears the sequence's selector
// histograms (both levels), which the scores pass and the filter fill.
__global__ __launch_bounds__(256) void score_reduce_f32(
    const float2* __restrict__ stats, int nchunks, const int32_t* __restrict__ ctx_len, int cap,
    int H, float* __restrict__ lse2, float* __restrict__ lse_out, uint32_t* __restrict__ hist) {
  const int b = blockIdx.x;
  if (hist != nullptr)
    for (int i = threadIdx.x; i < kHistRow; i += blockDim.x) hist[(size_t)b * kHistRow + i] = 0u;
  const int N = clamp_ctx(ctx_len, b, cap);
  const int nc = (N + kF32Chunk - 1) / kF32Chunk;
  __shared__ float2 red[8][32];
  const float L = reduce_chunk_stats(stats + (size_t)b * nchunks * kMaxHeads, nc, red);
  if (threadIdx.x < 32) {
    const int h = threadIdx.x;
    lse2[b * kMaxHeads + h] = (h < H) ? L : INFINITY;
    if (lse_out != nullptr && h < H) lse_out[b * H + h] = L * 0.69314718055994531f;
  }
}

// Both MFMA passes; hist null: no selector histogram.
template <bool kFp8>
void launch_score_mfma(const hs2_attn_desc& d, const void* q, const void* k, int64_t kv_stride,
                       const int32_t* ctx_len, int cap, float* scores, float* lse, float2* stats,
                       int nchunks1, float c2, uint32_t* hist, hipStream_t st) {
  const auto* qq = static_cast<const uint16_t*>(q);
  score_p1_bf16<kFp8><<<dim3(nchunks1, d.batch), 64 * kP1Waves, 0, st>>>(
      qq, k, kv_stride, ctx_len, cap, d.n_heads, c2, stats, nchunks1, hist);
  const dim3 g2((cap + kP2Chunk - 1) / kP2Chunk, d.batch);
  if (hist != nullptr)
    score_p2_bf16<kFp8, true><<<g2, 64 * kP2Waves, 0, st>>>(
        qq, k, kv_stride, ctx_len, cap, d.n_heads, c2, stats, nchunks1, scores, cap, lse, hist,
        d.window);
  else
    score_p2_bf16<kFp8, false><<<g2, 64 * kP2Waves, 0, st>>>(
        qq, k, kv_stride, ctx_len, cap, d.n_heads, c2, stats, nchunks1, scores, cap, lse, nullptr,
        d.window);
}

}  // namespace

hipError_t launch_score_full(const hs2_attn_desc& d, const void* q, const void* k, const void* v,
                             int64_t kv_stride, const int32_t* ctx_len, int cap, float* scores,
                             float* o_full, float* lse, char* ws, hipStream_t st) {
  const ScoreWs w = score_ws(d, cap);
  float2* stats = reinterpret_cast<float2*>(ws + w.stats_off);
  float* o_part = reinterpret_cast<float*>(ws + w.opart_off);
  const int nchunks2 = (cap + kP2Chunk - 1) / kP2Chunk;
  if (d.dtype == HS2_F32) {
    float* lse2 = reinterpret_cast<float*>(ws + w.lse2_off);
    const int nchunks1 = score_nchunks1(d, cap);
    const auto* qf = static_cast<const float*>(q);
    const auto* kf = static_cast<const float*>(k);
    launch_score_f32<0>(dim3(nchunks1, d.batch), st, qf, kf, kv_stride, ctx_len, cap, d.n_heads,
                        d.sm_scale * 1.4426950408889634f, stats, nchunks1, nullptr, nullptr, 0);
    score_reduce_f32<<<d.batch, 256, 0, st>>>(stats, nchunks1, ctx_len, cap, d.n_heads, lse2, lse,
                                              nullptr);
    score_full_f32<<<dim3(nchunks2, d.batch), 256, 0, st>>>(
        qf, kf, static_cast<const float*>(v), kv_stride, ctx_len, cap, d.n_heads,
        d.sm_scale * 1.4426950408889634f, lse2, scores, cap, o_part, nchunks2);
    full_out_combine<<<dim3(d.n_heads, d.batch), 32 * kCombGroups, 0, st>>>(
        o_part, nchunks2, ctx_len, cap, d.n_heads, 1.f, o_full);
    return hipGetLastError();
  }
  const bool fp8 = d.dtype == HS2_FP8_E4M3;
  const float c2 = d.sm_scale * 1.4426950408889634f * (fp8 ? d.k_scale : 1.f);
  const int nchunks1 = score_nchunks1(d, cap);
  const auto* qq = static_cast<const uint16_t*>(q);
  const dim3 g1(nchunks1, d.batch), g2(nchunks2, d.batch);
  if (fp8) {
    score_p1_bf16<true><<<g1, 64 * kP1Waves, 0, st>>>(qq, k, kv_stride, ctx_len, cap, d.n_heads,
                                                      c2, stats, nchunks1, nullptr);
    score_p2_full<true><<<g2, 64 * kP2Waves, 0, st>>>(qq, k, v, kv_stride, ctx_len, cap,
                                                      d.n_heads, c2, stats, nchunks1, scores, cap,
                                                      lse, o_part, nchunks2);
  } else {
    score_p1_bf16<false><<<g1, 64 * kP1Waves, 0, st>>>(qq, k, kv_stride, ctx_len, cap, d.n_heads,
                                                       c2, stats, nchunks1, nullptr);
    score_p2_full<false><<<g2, 64 * kP2Waves, 0, st>>>(qq, k, v, kv_stride, ctx_len, cap,
                                                       d.n_heads, c2, stats, nchunks1, scores,
                                                       cap, lse, o_part, nchunks2);
  }
  full_out_combine<<<dim3(d.n_heads, d.batch), 32 * kCombGroups, 0, st>>>(
      o_part, nchunks2, ctx_len, cap, d.n_heads, fp8 ? d.v_scale : 1.f, o_full);
  return hipGetLastError();
}

hipError_t launch_score_decode(const hs2_attn_desc& d, const void* q, const void* k,
                               int64_t kv_stride, const int32_t* ctx_len, int cap,
                               float* scores, float* lse, char* ws, uint64_t* sync,
                               bool with_hist, hipStream_t st, const FilterArgs* filt,
                               bool* filtered) {
  if (filtered != nullptr) *filtered = false;
  const ScoreWs w = score_ws(d, cap);
  float2* stats = reinterpret_cast<float2*>(ws + w.stats_off);
  const float c2 = d.sm_scale * 1.4426950408889634f;
  const int nchunks1 = score_nchunks1(d, cap);
  if (d.dtype != HS2_F32) {
    uint32_t* hist = with_hist ? reinterpret_cast<uint32_t*>(ws + w.hist_off) : nullptr;
    int nwg = 0, chunk = 0;
    if (sync != nullptr && onepass_plan(d, cap, device_cu_count(), &nwg, &chunk)) {
      // The one-pass kernel builds the histogram only together with the filter.
      if (hist != nullptr && filt == nullptr) return hipErrorInvalidValue;
      if (filtered != nullptr) *filtered = hist != nullptr;
      return launch_score_onepass(d, q, k, kv_stride, ctx_len, cap, nwg, chunk,
                                  d.dtype == HS2_FP8_E4M3 ? c2 * d.k_scale : c2,
                                  reinterpret_cast<float*>(ws + w.op_off), sync, scores, lse,
                                  hist, filt, st);
    }
    if (d.dtype == HS2_FP8_E4M3)
      launch_score_mfma<true>(d, q, k, kv_stride, ctx_len, cap, scores, lse, stats, nchunks1,
                              c2 * d.k_scale, hist, st);
    else
      launch_score_mfma<false>(d, q, k, kv_stride, ctx_len, cap, scores, lse, stats, nchunks1,
                               c2, hist, st);
  } else {
    const dim3 grid(nchunks1, d.batch);
    const auto* qf = static_cast<const float*>(q);
    const auto* kf = static_cast<const float*>(k);
    uint32_t* hist = with_hist ? reinterpret_cast<uint32_t*>(ws + w.hist_off) : nullptr;
    launch_score_f32<0>(grid, st, qf, kf, kv_stride, ctx_len, cap, d.n_heads, c2, stats,
                        nchunks1, nullptr, nullptr, 0, hist);
    launch_score_f32<1>(grid, st, qf, kf, kv_stride, ctx_len, cap, d.n_heads, c2, stats,
                        nchunks1, lse, scores, cap, hist, d.window);
  }
  return hipGetLastError();
}

}  // namespace hs2
