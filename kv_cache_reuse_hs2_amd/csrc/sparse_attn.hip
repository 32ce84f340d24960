// Sparse attention over the selected keys plus the forced recent window.
//
// The sparse layers that follow a full-attention layer reuse its selection
// and read the same K/V cache; the 128 most recent tokens are always part of
// what they attend to ("HySparse2: How Xiaomi Split the Transformer to Fix
// Agent Prefill Costs", section "KV Reuse and Token-Level Sparse
// Selection").  For a query at position P of group g:
//   S = top_idx[g][0..cnt) ++ [max(0, P - window + 1), P]
//   o_h = sum_{j in S} softmax_S(sm_scale * q_h.k_j) v_j
//
// The selection (at most k_top + window keys) is split into 32-key segments;
// one workgroup gathers a segment's K and V rows into LDS, computes the
// 32 x H logits and its local softmax, and writes a partial (max, sum, o).
// A second kernel merges the partials of each query in segment order, so the
// result does not depend on scheduling.
#include "hs2_internal.h"

namespace hs2 {
namespace {

template <typename T>
__device__ __forceinline__ float ld_elem(const T* p, int i);
template <>
__device__ __forceinline__ float ld_elem<float>(const float* p, int i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p, int i) { return bf16_to_f32(p[i]); }

// Load 16 consecutive elements starting at p (16-B aligned) as fp32.
template <typename T>
__device__ __forceinline__ void load16(const T* p, float* dst);
template <>
__device__ __forceinline__ void load16<float>(const float* p, float* dst) {
  const float4* s = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = s[i];
    dst[4 * i] = v.x;
    dst[4 * i + 1] = v.y;
    dst[4 * i + 2] = v.z;
    dst[4 * i + 3] = v.w;
  }
}
template <>
__device__ __forceinline__ void load16<uint16_t>(const uint16_t* p, float* dst) {
  const u32x4* s = reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const u32x4 v = s[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dst[8 * i + 2 * e] = __uint_as_float(v[e] << 16);
      dst[8 * i + 2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
    }
  }
}

constexpr int kSeg = kSparseSeg;   // keys per workgroup
constexpr int kKPitch = kHeadDim + 4;  // LDS row pitch of K (bank spread)

template <typename T>
__global__ __launch_bounds__(256) void sparse_partial(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t kv_stride,
    const int32_t* __restrict__ ctx_len, int cap, const int32_t* __restrict__ top_idx,
    const int32_t* __restrict__ top_cnt, int n_q, int tile_q, int k_top, int window, int H,
    float sm_scale, float* __restrict__ part, float2* __restrict__ ml, int nseg) {
  const int seg = blockIdx.x;
  const int bq = blockIdx.y;
  const int b = bq / n_q, i = bq % n_q, g = i / tile_q;
  const int tiles = n_q / tile_q;
  const int t = threadIdx.x;
  const int N = clamp_ctx(ctx_len, b, cap);
  const int P = N - n_q + i;
  int cnt = 0, wlo = 0, wcnt = 0;
  if (P >= 0) {
    cnt = top_cnt[b * tiles + g];
    cnt = cnt < 0 ? 0 : (cnt > k_top ? k_top : cnt);
    wlo = max(0, P - window + 1);
    wcnt = P - wlo + 1;
  }
  const int S = cnt + wcnt;
  const int s0 = seg * kSeg;
  float2* mlo = ml + ((size_t)bq * nseg + seg) * H;
  if (s0 >= S) {
    if (t < H) mlo[t] = make_float2(-INFINITY, 0.f);
    return;
  }
  const int nk = min(kSeg, S - s0);

  __shared__ float qs[kMaxHeads][kHeadDim];
  __shared__ float ks[kSeg][kKPitch];
  __shared__ float vs[kSeg][kHeadDim];
  __shared__ float ps[kSeg][kMaxHeads];
  __shared__ int kidx[kSeg];

  if (t < kSeg) {
    int idx = 0;
    if (t < nk) {
      const int p = s0 + t;
      idx = p < cnt ? top_idx[(size_t)(b * tiles + g) * k_top + p] : wlo + (p - cnt);
      idx = idx < 0 ? 0 : (idx >= N ? N - 1 : idx);  // memory safety only
    }
    kidx[t] = idx;
  }
  const T* qb = q + (size_t)bq * H * kHeadDim;
  for (int e = t; e < kMaxHeads * kHeadDim / 16; e += blockDim.x) {
    const int h = e / (kHeadDim / 16), c = (e % (kHeadDim / 16)) * 16;
    float tmp[16];
    if (h < H) {
      load16<T>(qb + h * kHeadDim + c, tmp);
    } else {
#pragma unroll
      for (int x = 0; x < 16; ++x) tmp[x] = 0.f;
    }
#pragma unroll
    for (int x = 0; x < 16; ++x) qs[h][c + x] = tmp[x];
  }
  __syncthreads();
  // Gather K and V rows: 32 rows x 8 pieces of 16 elements = 256 pieces each.
  {
    const int row = t >> 3, c = (t & 7) * 16;
    float tk[16], tv[16];
    const size_t off = (size_t)b * kv_stride + (size_t)kidx[row] * kHeadDim + c;
    load16<T>(k + off, tk);
    load16<T>(v + off, tv);
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      ks[row][c + x] = tk[x];
      vs[row][c + x] = tv[x];
    }
  }
  __syncthreads();
  // Logits: thread (key kx, heads hg, hg+8, hg+16, hg+24).
  {
    const int kx = t & 31, hg = t >> 5;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int d = 0; d < kHeadDim; d += 4) {
      const float4 kv = *reinterpret_cast<const float4*>(&ks[kx][d]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 qv = *reinterpret_cast<const float4*>(&qs[hg + 8 * u][d]);
        acc[u] = fmaf(qv.x, kv.x, acc[u]);
        acc[u] = fmaf(qv.y, kv.y, acc[u]);
        acc[u] = fmaf(qv.z, kv.z, acc[u]);
        acc[u] = fmaf(qv.w, kv.w, acc[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) ps[kx][hg + 8 * u] = (kx < nk) ? acc[u] * sm_scale : -INFINITY;
  }
  __syncthreads();
  // Segment-local softmax per head.
  if (t < kMaxHeads) {
    float m = -INFINITY;
    for (int x = 0; x < nk; ++x) m = fmaxf(m, ps[x][t]);
    float l = 0.f;
    for (int x = 0; x < kSeg; ++x) {
      const float p = (x < nk) ? __expf(ps[x][t] - m) : 0.f;
      ps[x][t] = p;
      l += p;
    }
    if (t < H) mlo[t] = make_float2(m, l);
  }
  __syncthreads();
  // P V: thread (dim d, heads 16*hh .. 16*hh+15).
  {
    const int d = t & (kHeadDim - 1), hh = t >> 7;
    float o[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) o[u] = 0.f;
    for (int x = 0; x < nk; ++x) {
      const float vx = vs[x][d];
#pragma unroll
      for (int u = 0; u < 16; u += 4) {
        const float4 p = *reinterpret_cast<const float4*>(&ps[x][16 * hh + u]);
        o[u] = fmaf(p.x, vx, o[u]);
        o[u + 1] = fmaf(p.y, vx, o[u + 1]);
        o[u + 2] = fmaf(p.z, vx, o[u + 2]);
        o[u + 3] = fmaf(p.w, vx, o[u + 3]);
      }
    }
    float* po = part + (((size_t)bq * nseg + seg) * H) * kHeadDim;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int h = 16 * hh + u;
      if (h < H) po[(size_t)h * kHeadDim + d] = o[u];
    }
  }
}

// Merge the segment partials of each query: o = sum_s e^(m_s-M) o_s / sum_s e^(m_s-M) l_s.
__global__ __launch_bounds__(256) void sparse_combine(const float* __restrict__ part,
                                                      const float2* __restrict__ ml, int nseg,
                                                      int H, float* __restrict__ o,
                                                      float* __restrict__ lse) {
  const int bq = blockIdx.x;
  const int d = threadIdx.x & (kHeadDim - 1), hh = threadIdx.x >> 7;
  const float2* mlq = ml + (size_t)bq * nseg * H;
  const float* pq = part + (size_t)bq * nseg * H * kHeadDim;
  for (int h = hh; h < H; h += 2) {
    float M = -INFINITY;
    for (int s = 0; s < nseg; ++s) {
      const float2 x = mlq[(size_t)s * H + h];
      if (x.y > 0.f) M = fmaxf(M, x.x);
    }
    float den = 0.f, num = 0.f;
    for (int s = 0; s < nseg; ++s) {
      const float2 x = mlq[(size_t)s * H + h];
      if (x.y > 0.f) {
        const float w = __expf(x.x - M);
        den = fmaf(w, x.y, den);
        num = fmaf(w, pq[((size_t)s * H + h) * kHeadDim + d], num);
      }
    }
    o[((size_t)bq * H + h) * kHeadDim + d] = den > 0.f ? num / den : 0.f;
    if (lse != nullptr && d == 0) lse[(size_t)bq * H + h] = den > 0.f ? M + __logf(den) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_sparse(const hs2_attn_desc& d, const void* q, const void* k, const void* v,
                         int64_t kv_stride, const int32_t* ctx_len, int cap,
                         const int32_t* top_idx, const int32_t* top_cnt, float* o, float* lse,
                         char* ws, hipStream_t st) {
  const SparseWs w = sparse_ws(d);
  float* part = reinterpret_cast<float*>(ws + w.part_off);
  float2* ml = reinterpret_cast<float2*>(ws + w.ml_off);
  int nseg = sparse_segments(d);
  if (nseg < 1) nseg = 1;
  const dim3 grid(nseg, d.batch * d.n_q);
  if (d.dtype == HS2_BF16) {
    sparse_partial<uint16_t><<<grid, 256, 0, st>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
        static_cast<const uint16_t*>(v), kv_stride, ctx_len, cap, top_idx, top_cnt, d.n_q,
        d.tile_q, d.k_top, d.window, d.n_heads, d.sm_scale, part, ml, nseg);
  } else {
    sparse_partial<float><<<grid, 256, 0, st>>>(
        static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
        kv_stride, ctx_len, cap, top_idx, top_cnt, d.n_q, d.tile_q, d.k_top, d.window,
        d.n_heads, d.sm_scale, part, ml, nseg);
  }
  sparse_combine<<<d.batch * d.n_q, 256, 0, st>>>(part, ml, nseg, d.n_heads, o, lse);
  return hipGetLastError();
}

}  // namespace hs2
