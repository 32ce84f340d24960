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
// The selection (at most k_top + window keys) is cut into segments; one
// workgroup gathers a segment's K and V rows and writes a partial
// (max, sum, o) per head in base 2; sparse_combine merges the partials of a
// query in segment order, so results do not depend on scheduling.
//
// bf16: 128-key segments, one wave per 32 keys.  QK^T is eight
// v_mfma_f32_32x32x16_bf16 with the gathered K rows as the A operand (a lane
// reads 16 contiguous bytes of one row per step), so each lane owns one head
// over 16 keys and the wave's softmax statistics stay in-lane.  The
// probabilities feed the PV product straight from those registers (A operand,
// keys in the order the QK^T result holds them), split into a bf16 high and
// low part so that the sum keeps about fp32 accuracy; V is transposed
// through LDS into the matching B layout.  The four waves are merged in LDS in
// a fixed order.
// E4M3 caches take the same path: the gather widens the bytes to bf16 in
// registers (exact), the K scale multiplies the logit scale and the V scale
// the merged output (o is linear in V).
// fp32: 32-key segments on VALU.
#include "hs2_internal.h"
#include "select_core.h"

namespace hs2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// Selection-set geometry of one query.
struct QueryGeom {
  int N, cnt, wlo, S;
};

__device__ __forceinline__ QueryGeom query_geom(const int32_t* ctx_len, const int32_t* top_cnt,
                                                int cap, int b, int i, int g, int tiles, int n_q,
                                                int k_top, int window) {
  QueryGeom q{};
  q.N = clamp_ctx(ctx_len, b, cap);
  const int P = q.N - n_q + i;
  int wcnt = 0;
  if (P >= 0) {
    int c = top_cnt[b * tiles + g];
    q.cnt = c < 0 ? 0 : (c > k_top ? k_top : c);
    q.wlo = max(0, P - window + 1);
    wcnt = P - q.wlo + 1;
  }
  q.S = q.cnt + wcnt;
  return q;
}

// Key index of selection position p (0 <= p < S), clamped into the cache for
// memory safety (selector output is always inside it).
__device__ __forceinline__ int sel_key(const QueryGeom& q, const int32_t* top_row, int p) {
  int idx = p < q.cnt ? top_row[p] : q.wlo + (p - q.cnt);
  return idx < 0 ? 0 : (idx >= q.N ? q.N - 1 : idx);
}

// ---------------------------------------------------------------------------
// bf16, MFMA.

constexpr int kSegWaves = 4;
static_assert(kSegB == 32 * kSegWaves, "keys per workgroup");
constexpr int kVtPitch = 40;           // bf16 per transposed V row (32 keys + pad)

// LDS of one segment.
struct SegLds {
  uint16_t vt[kSegWaves][kHeadDim][kVtPitch];
  float s_m[kSegWaves][32], s_l[kSegWaves][32];
  float s_sc[kSegWaves][32];  // per wave and head: 2^(wave max - workgroup max)
  float s_o[kSegWaves][32][kHeadDim + 4];
};

// Gather of the segment starting at selection position s0 (sequence b):
// waves 0..kSegWaves-1 load 32 keys each, K rows into kr as bf16 (the A
// operand of QK^T: lane = key r32, dims step_dim(e, hh) in step e) and V rows
// transposed into L.vt (vt[wave][d][key]).  key_at(p) gives the cache index
// of selection position p < qg.S.  Called by every thread; other waves do
// nothing.
template <bool kFp8, typename KeyAt>
__device__ __forceinline__ void segment_gather_bf16(const void* __restrict__ k,
                                                    const void* __restrict__ v,
                                                    int64_t kv_stride, int b,
                                                    const QueryGeom& qg, int s0, KeyAt key_at,
                                                    SegLds& L, u32x4 (&kr)[8]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  if (wave >= kSegWaves) return;
  const int pw = s0 + 32 * wave;  // first selection position of this wave
  const int idx = key_at((pw + r32 < qg.S) ? pw + r32 : s0);
  const size_t rowoff =
      ((size_t)b * kv_stride + (size_t)idx * kHeadDim) * kv_elem_bytes<kFp8>();
  const char* krow = static_cast<const char*>(k) + rowoff;
  const char* vrow = static_cast<const char*>(v) + rowoff;
  u32x4 vr[8];  // bf16 V of dims 64hh + 8e .. +8
  if constexpr (kFp8) {
    // K: pieces 2i + hh (dims 32i + 16hh .. +16); V: dims 64hh + 16i .. +16.
    const u32x4* kp = reinterpret_cast<const u32x4*>(krow) + hh;
    const u32x4* vp = reinterpret_cast<const u32x4*>(vrow + 64 * hh);
    u32x4 kb8[4], vb8[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kb8[i] = kp[2 * i];
      vb8[i] = vp[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kr[2 * i] = e4m3x8_to_bf16x8(kb8[i][0], kb8[i][1]);
      kr[2 * i + 1] = e4m3x8_to_bf16x8(kb8[i][2], kb8[i][3]);
      vr[2 * i] = e4m3x8_to_bf16x8(vb8[i][0], vb8[i][1]);
      vr[2 * i + 1] = e4m3x8_to_bf16x8(vb8[i][2], vb8[i][3]);
    }
  } else {
    const u32x4* kp = reinterpret_cast<const u32x4*>(krow) + hh;
    const u32x4* vp = reinterpret_cast<const u32x4*>(vrow + 128 * hh);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kr[e] = kp[2 * e];
      vr[e] = vp[e];
    }
  }
  // V transposed into LDS: vt[wave][d][key], key = r32, d = 64*hh + 8*e + j.
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      L.vt[wave][64 * hh + 8 * e + 2 * j][r32] = (uint16_t)(vr[e][j] & 0xFFFFu);
      L.vt[wave][64 * hh + 8 * e + 2 * j + 1][r32] = (uint16_t)(vr[e][j] >> 16);
    }
}

// Q^T of one query as the B operand of QK^T (lane: head r32, dims
// step_dim(e, hh) in step e; heads >= H and waves past the segment's zero).
// Loaded by the callers ahead of the gather, so that its round trip overlaps
// the gather's (or the selection's).
template <bool kFp8>
__device__ __forceinline__ void load_q_segment(const uint16_t* __restrict__ qb, int H,
                                               bf16x8_t (&qreg)[8]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    u32x4 xq = {0u, 0u, 0u, 0u};
    if (wave < kSegWaves && r32 < H)
      xq = *reinterpret_cast<const u32x4*>(qb + r32 * kHeadDim + step_dim<kFp8>(e, hh));
    qreg[e] = as_bf16x8(xq);
  }
}

// Partial of one query over the gathered segment (kr, L.vt): (max, sum) per
// head to mlo[H] and o to po[H][D]; qreg holds the query (load_q_segment).
// Called by every thread of the workgroup, after segment_gather_bf16; its
// barriers also order the gather's LDS writes before the PV reads.  The LDS
// statistics and partials are free again when it returns.
template <bool kFp8>
__device__ __forceinline__ void segment_query_bf16(const bf16x8_t (&qreg)[8], int H,
                                                   float c2, const QueryGeom& qg, int s0,
                                                   const u32x4 (&kr)[8], SegLds& L,
                                                   float* __restrict__ po,
                                                   float2* __restrict__ mlo) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  const bool active = wave < kSegWaves;
  const int pw = s0 + 32 * wave;  // first selection position of this wave
  const bool wave_live = active && pw < qg.S;
  float x[16];
  if (active) {
    f32x16_t acc = {};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr[e]), qreg[e], acc, 0, 0, 0);
    // acc[r]: head r32, key 8*(r/4) + 4*hh + r%4 of this wave's 32.
    float m = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * hh + (r & 3);
      x[r] = (pw + key < qg.S) ? acc[r] * c2 : -INFINITY;
      m = fmaxf(m, x[r]);
    }
    m = fmaxf(m, __shfl_xor(m, 32));
    const float mref = (m == -INFINITY) ? 0.f : m;
    float l = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[r] = fast_exp2(x[r] - mref);
      l += x[r];
    }
    l += __shfl_xor(l, 32);
    if (hh == 0) {
      L.s_m[wave][r32] = wave_live ? m : -INFINITY;
      L.s_l[wave][r32] = wave_live ? l : 0.f;
    }
  }
  __syncthreads();
  if (active) {
    // This wave's rescale factors, one head per lane of the low half, read
    // back four heads at a time (they do not depend on P V, so their LDS
    // round trips overlap the MFMAs below).
    if (hh == 0) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kSegWaves; ++w) M = fmaxf(M, L.s_m[w][r32]);
      const float mw = L.s_m[wave][r32];
      L.s_sc[wave][r32] = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
    }
    wave_lds_sync();
    float sc[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 x = *reinterpret_cast<const float4*>(&L.s_sc[wave][8 * g + 4 * hh]);
      sc[4 * g] = x.x;
      sc[4 * g + 1] = x.y;
      sc[4 * g + 2] = x.z;
      sc[4 * g + 3] = x.w;
    }
    // P V for this wave's 32 keys: k-step s covers the keys of registers
    // 8s..8s+7, i.e. {16s + 4hh + 0..3} and {16s + 8 + 4hh + 0..3}.
    f32x16_t o[4] = {{}, {}, {}, {}};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 ahi, alo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = x[8 * s + 2 * j], p1 = x[8 * s + 2 * j + 1];
        const uint16_t h0 = f32_to_bf16_rne(p0), h1 = f32_to_bf16_rne(p1);
        const uint16_t l0 = f32_to_bf16_rne(p0 - bf16_to_f32(h0));
        const uint16_t l1 = f32_to_bf16_rne(p1 - bf16_to_f32(h1));
        ahi[j] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        alo[j] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint16_t* row = &L.vt[wave][32 * t + r32][0];
        const uint2 lo4 = *reinterpret_cast<const uint2*>(row + 16 * s + 4 * hh);
        const uint2 hi4 = *reinterpret_cast<const uint2*>(row + 16 * s + 8 + 4 * hh);
        const u32x4 bv = {lo4.x, lo4.y, hi4.x, hi4.y};
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ahi), as_bf16x8(bv), o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(alo), as_bf16x8(bv), o[t], 0, 0, 0);
      }
    }
    // o[t][r]: head 8*(r/4) + 4*hh + r%4, dim 32*t + r32, relative to this
    // wave's max; rescale to the workgroup max and stage for the merge.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int h = 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
      for (int t = 0; t < 4; ++t) L.s_o[wave][h][32 * t + r32] = o[t][r] * sc[r];
    }
  }
  __syncthreads();
  // Merge the waves in order, four outputs of a thread at a time so that
  // their LDS reads are in flight together.
  for (int e0 = threadIdx.x; e0 < 32 * kHeadDim; e0 += 4 * blockDim.x) {
    float acc_o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * blockDim.x;
      const int h = e / kHeadDim, d = e % kHeadDim;
      acc_o[u] = 0.f;
      if (e < 32 * kHeadDim)
#pragma unroll
        for (int w = 0; w < kSegWaves; ++w) acc_o[u] += L.s_o[w][h][d];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * blockDim.x;
      const int h = e / kHeadDim, d = e % kHeadDim;
      if (e < 32 * kHeadDim && h < H) po[(size_t)h * kHeadDim + d] = acc_o[u];
    }
  }
  if (threadIdx.x < H) {
    const int h = threadIdx.x;
    float M = -INFINITY;
    for (int w = 0; w < kSegWaves; ++w) M = fmaxf(M, L.s_m[w][h]);
    float Ls = 0.f;
    for (int w = 0; w < kSegWaves; ++w)
      if (L.s_m[w][h] != -INFINITY) Ls += L.s_l[w][h] * fast_exp2(L.s_m[w][h] - M);
    mlo[h] = make_float2(M, Ls);
  }
  __syncthreads();
}

// Gather and partial of one query (one sparse layer).
template <bool kFp8, typename KeyAt>
__device__ __forceinline__ void segment_partial_bf16(
    const bf16x8_t (&qreg)[8], const void* __restrict__ k, const void* __restrict__ v,
    int64_t kv_stride, int b, int H, float c2, const QueryGeom& qg, int s0,
    KeyAt key_at, SegLds& L, float* __restrict__ po, float2* __restrict__ mlo) {
  u32x4 kr[8];
  segment_gather_bf16<kFp8>(k, v, kv_stride, b, qg, s0, key_at, L, kr);
  segment_query_bf16<kFp8>(qreg, H, c2, qg, s0, kr, L, po, mlo);
}

template <bool kFp8>
__global__ __launch_bounds__(64 * kSegWaves) void sparse_partial_bf16(
    const uint16_t* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    int64_t kv_stride, const int32_t* __restrict__ ctx_len,
    int cap, const int32_t* __restrict__ top_idx, const int32_t* __restrict__ top_cnt, int n_q,
    int tile_q, int k_top, int window, int H, float c2, float* __restrict__ part,
    float2* __restrict__ ml, int nseg) {
  __shared__ SegLds lds;
  const int seg = blockIdx.x, bq = blockIdx.y;
  const int b = bq / n_q, i = bq % n_q, g = i / tile_q, tiles = n_q / tile_q;
  const QueryGeom qg = query_geom(ctx_len, top_cnt, cap, b, i, g, tiles, n_q, k_top, window);
  const int s0 = seg * kSegB;
  float2* mlo = ml + ((size_t)bq * nseg + seg) * H;
  if (s0 >= qg.S) {
    if (threadIdx.x < H) mlo[threadIdx.x] = make_float2(-INFINITY, 0.f);
    return;
  }
  const int32_t* top_row = top_idx + (size_t)(b * tiles + g) * k_top;
  bf16x8_t qreg[8];
  load_q_segment<kFp8>(q + (size_t)bq * H * kHeadDim, H, qreg);
  segment_partial_bf16<kFp8>(qreg, k, v, kv_stride, b, H, c2, qg, s0,
                             [&](int p) { return sel_key(qg, top_row, p); }, lds,
                             part + ((size_t)bq * nseg + seg) * H * kHeadDim, mlo);
}

// ---------------------------------------------------------------------------
// Several sparse layers after one full layer (decode): the layers share
// the selection and the K/V cache, so each workgroup gathers its segment once
// and runs every layer's query over it.  Partials are laid out as if the
// layers were extra queries (row l*B + b), so sparse_combine merges them.
template <bool kFp8>
__global__ __launch_bounds__(64 * kSegWaves) void sparse_layers_bf16(
    const uint16_t* __restrict__ q_layers, const void* __restrict__ k,
    const void* __restrict__ v, int64_t kv_stride, const int32_t* __restrict__ ctx_len,
    int cap, const int32_t* __restrict__ top_idx, const int32_t* __restrict__ top_cnt, int B,
    int k_top, int window, int H, float c2, int n_layers, float* __restrict__ part,
    float2* __restrict__ ml, int nseg) {
  __shared__ SegLds lds;
  const int seg = blockIdx.x, b = blockIdx.y;  // one query per sequence
  const QueryGeom qg = query_geom(ctx_len, top_cnt, cap, b, 0, 0, 1, 1, k_top, window);
  const int s0 = seg * kSegB;
  if (s0 >= qg.S) {
    if (threadIdx.x < H)
      for (int l = 0; l < n_layers; ++l)
        ml[((size_t)(l * B + b) * nseg + seg) * H + threadIdx.x] = make_float2(-INFINITY, 0.f);
    return;
  }
  const int32_t* top_row = top_idx + (size_t)b * k_top;
  u32x4 kr[8];
  segment_gather_bf16<kFp8>(k, v, kv_stride, b, qg, s0,
                            [&](int p) { return sel_key(qg, top_row, p); }, lds, kr);
  for (int l = 0; l < n_layers; ++l) {
    const int row = l * B + b;
    bf16x8_t qreg[8];
    load_q_segment<kFp8>(q_layers + (size_t)row * H * kHeadDim, H, qreg);
    segment_query_bf16<kFp8>(qreg, H, c2, qg, s0, kr, lds,
                             part + ((size_t)row * nseg + seg) * H * kHeadDim,
                             ml + ((size_t)row * nseg + seg) * H);
  }
}

// ---------------------------------------------------------------------------
// Fused decode tail (bf16): the final selection of sequence blockIdx.y and
// the partial of segment blockIdx.x, in one launch.  Every workgroup of the
// sequence resolves the same selection from the filter's candidate lists
// into LDS (the first one also writes top_idx and top_cnt), then gathers its
// segment exactly as sparse_partial_bf16 would from top_idx.

constexpr int kTailThreads = 1024;

union TailLds {
  struct {
    uint32_t h[256];
    uint2 stage[kStage];
    uint32_t pre[kMaxSlices + 1];
    uint32_t chunk_wins[2 * kStage / 64];
    uint32_t scratch[16];
    uint32_t res[6];
  } sel;
  SegLds seg;
};

template <bool kFp8>
__global__ __launch_bounds__(kTailThreads) void decode_tail_bf16(
    const uint16_t* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    int64_t kv_stride, const int32_t* __restrict__ ctx_len,
    int cap, int k_top, int window, int H, float c2, const uint32_t* __restrict__ hist,
    const uint32_t* __restrict__ cnt, const uint32_t* __restrict__ meta,
    const uint2* __restrict__ list, int nslices, int32_t* __restrict__ top_idx,
    int32_t* __restrict__ top_cnt, float* __restrict__ part, float2* __restrict__ ml, int nseg) {
  __shared__ __attribute__((aligned(16))) TailLds lds;
  __shared__ int32_t win[kMaxTop];
  const int seg = blockIdx.x, b = blockIdx.y;  // one query per sequence
  // The query's loads go out first and complete during the selection.
  bf16x8_t qreg[8];
  load_q_segment<kFp8>(q + (size_t)b * H * kHeadDim, H, qreg);
  const RowGeom g = row_geom(ctx_len, cap, b, 1, 1, 1, k_top, window);
  const int n = final_select_row<kTailThreads>(
      b, g, k_top, hist, cnt, meta, list, nslices, seg == 0 ? top_idx + (size_t)b * k_top : nullptr,
      win,
      FinalLds{lds.sel.h, lds.sel.pre, lds.sel.chunk_wins, lds.sel.scratch, lds.sel.res,
               lds.sel.stage});
  if (seg == 0 && threadIdx.x == 0) top_cnt[b] = n;
  // Selection geometry of the query, as query_geom reads it back from top_cnt.
  QueryGeom qg{};
  qg.N = clamp_ctx(ctx_len, b, cap);
  const int P = qg.N - 1;
  if (P >= 0) {
    qg.cnt = n;
    qg.wlo = max(0, P - window + 1);
    qg.S = n + (P - qg.wlo + 1);
  }
  const int s0 = seg * kSegB;
  float2* mlo = ml + ((size_t)b * nseg + seg) * H;
  if (s0 >= qg.S) {
    if (threadIdx.x < H) mlo[threadIdx.x] = make_float2(-INFINITY, 0.f);
    return;
  }
  auto key_at = [&](int p) {
    const int idx = p < qg.cnt ? win[p] : qg.wlo + (p - qg.cnt);
    return idx < 0 ? 0 : (idx >= qg.N ? qg.N - 1 : idx);
  };
  segment_partial_bf16<kFp8>(qreg, k, v, kv_stride, b, H, c2, qg, s0, key_at, lds.seg,
                             part + ((size_t)b * nseg + seg) * H * kHeadDim, mlo);
}

// ---------------------------------------------------------------------------
// fp32, VALU.

constexpr int kSegF = kSparseSeg;     // keys per workgroup
constexpr int kKPitch = kHeadDim + 4;  // LDS row pitch of K (bank spread)

__global__ __launch_bounds__(256) void sparse_partial_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    int64_t kv_stride, const int32_t* __restrict__ ctx_len, int cap,
    const int32_t* __restrict__ top_idx, const int32_t* __restrict__ top_cnt, int n_q, int tile_q,
    int k_top, int window, int H, float c2, float* __restrict__ part, float2* __restrict__ ml,
    int nseg) {
  const int seg = blockIdx.x, bq = blockIdx.y;
  const int b = bq / n_q, i = bq % n_q, g = i / tile_q, tiles = n_q / tile_q;
  const int t = threadIdx.x;
  const QueryGeom qg = query_geom(ctx_len, top_cnt, cap, b, i, g, tiles, n_q, k_top, window);
  const int s0 = seg * kSegF;
  float2* mlo = ml + ((size_t)bq * nseg + seg) * H;
  if (s0 >= qg.S) {
    if (t < H) mlo[t] = make_float2(-INFINITY, 0.f);
    return;
  }
  const int nk = min(kSegF, qg.S - s0);
  __shared__ float qs[kMaxHeads][kHeadDim];
  __shared__ float ks[kSegF][kKPitch];
  __shared__ float vs[kSegF][kHeadDim];
  __shared__ float ps[kSegF][kMaxHeads];
  __shared__ int kidx[kSegF];
  const int32_t* top_row = top_idx + (size_t)(b * tiles + g) * k_top;
  if (t < kSegF) kidx[t] = sel_key(qg, top_row, s0 + (t < nk ? t : 0));
  const float* qb = q + (size_t)bq * H * kHeadDim;
  for (int e = t; e < kMaxHeads * kHeadDim / 4; e += blockDim.x) {
    const int h = e / (kHeadDim / 4), c = (e % (kHeadDim / 4)) * 4;
    const float4 qv = h < H ? *reinterpret_cast<const float4*>(qb + h * kHeadDim + c)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(&qs[h][c]) = qv;
  }
  __syncthreads();
  {
    const int row = t >> 3, c = (t & 7) * 16;
    const size_t off = (size_t)b * kv_stride + (size_t)kidx[row] * kHeadDim + c;
#pragma unroll
    for (int x4 = 0; x4 < 4; ++x4) {
      *reinterpret_cast<float4*>(&ks[row][c + 4 * x4]) = reinterpret_cast<const float4*>(k + off)[x4];
      *reinterpret_cast<float4*>(&vs[row][c + 4 * x4]) = reinterpret_cast<const float4*>(v + off)[x4];
    }
  }
  __syncthreads();
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
    for (int u = 0; u < 4; ++u) ps[kx][hg + 8 * u] = (kx < nk) ? acc[u] * c2 : -INFINITY;
  }
  __syncthreads();
  if (t < kMaxHeads) {
    float m = -INFINITY;
    for (int x = 0; x < nk; ++x) m = fmaxf(m, ps[x][t]);
    float l = 0.f;
    for (int x = 0; x < kSegF; ++x) {
      const float p = (x < nk) ? fast_exp2(ps[x][t] - m) : 0.f;
      ps[x][t] = p;
      l += p;
    }
    if (t < H) mlo[t] = make_float2(m, l);
  }
  __syncthreads();
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
    float* po = part + ((size_t)bq * nseg + seg) * H * kHeadDim;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int h = 16 * hh + u;
      if (h < H) po[(size_t)h * kHeadDim + d] = o[u];
    }
  }
}

// ---------------------------------------------------------------------------
// Merge the segment partials of one (query, head): o = v_scale * sum_s
// 2^(m_s-M) o_s / sum_s 2^(m_s-M) l_s, segments taken in order (v_scale is
// the V cache scale of E4M3 caches, else 1).  One workgroup per (query, head),
// one thread per output dimension.  Up to kCombRegs segments are held in
// registers (launch_combine picks 16 for the MFMA paths, 9 segments at the
// usual budget, and 40 for the fp32 path's 36); more go through a loop.
template <int kCombRegs>
__global__ __launch_bounds__(kHeadDim) void sparse_combine(const float* __restrict__ part,
                                                           const float2* __restrict__ ml, int nseg,
                                                           int H, float v_scale,
                                                           float* __restrict__ o,
                                                           float* __restrict__ lse) {
  const int h = blockIdx.x, bq = blockIdx.y, d = threadIdx.x;
  const float2* mlq = ml + (size_t)bq * nseg * H + h;
  const float* pq = part + ((size_t)bq * nseg * H + h) * kHeadDim + d;
  // A segment with no keys (l == 0) has no partial output written, and is
  // masked by a select, never multiplied (its memory may hold anything).
  float den = 0.f, num = 0.f, M = -INFINITY;
  if (nseg <= kCombRegs) {
    // Every load at once (one memory round trip), then the same arithmetic
    // as the loop below.  The (max, sum) pairs, the same for every thread,
    // are loaded one per thread and shared through LDS (as scalar loads they
    // would need more scalar registers than there are).
    __shared__ float2 s_ml[kCombRegs];
    if (d < nseg) s_ml[d] = mlq[(size_t)d * H];
    // Partials through one buffer resource with per-segment vector offsets
    // (64-bit addresses per segment would also crowd the scalar registers).
    // Past the last segment the buffer loads return zero (never used).
    float pv[kCombRegs];
    const float* p0 = part + ((size_t)bq * nseg * H + h) * kHeadDim;  // uniform
    const uint32_t seg_bytes = (uint32_t)(H * kHeadDim * sizeof(float));
    const __amdgpu_buffer_rsrc_t rp = buffer_rsrc(p0, (uint32_t)nseg * seg_bytes);
#pragma unroll
    for (int s = 0; s < kCombRegs; ++s)
      pv[s] = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(rp, s * seg_bytes + d * (int)sizeof(float), 0, 0));
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kCombRegs; ++s)
      if (s < nseg && s_ml[s].y > 0.f) M = fmaxf(M, s_ml[s].x);
#pragma unroll
    for (int s = 0; s < kCombRegs; ++s)
      if (s < nseg) {
        const float2 x = s_ml[s];
        const bool live = x.y > 0.f;
        const float w = live ? fast_exp2(x.x - M) : 0.f;
        den = fmaf(w, live ? x.y : 0.f, den);
        num = live ? fmaf(w, pv[s], num) : num;
      }
  } else {
    for (int s = 0; s < nseg; ++s) {
      const float2 x = mlq[(size_t)s * H];
      if (x.y > 0.f) M = fmaxf(M, x.x);
    }
    // Loads are unconditional so that they can be issued together.
#pragma unroll 8
    for (int s = 0; s < nseg; ++s) {
      const float2 x = mlq[(size_t)s * H];
      const float pv = pq[(size_t)s * H * kHeadDim];
      const bool live = x.y > 0.f;
      const float w = live ? fast_exp2(x.x - M) : 0.f;
      den = fmaf(w, live ? x.y : 0.f, den);
      num = live ? fmaf(w, pv, num) : num;
    }
  }
  o[((size_t)bq * H + h) * kHeadDim + d] = den > 0.f ? num / den * v_scale : 0.f;
  if (lse != nullptr && d == 0)
    lse[(size_t)bq * H + h] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
}

void launch_combine(dim3 grid, hipStream_t st, const float* part, const float2* ml, int nseg,
                    int H, float v_scale, float* o, float* lse) {
  if (nseg <= 16)
    sparse_combine<16><<<grid, kHeadDim, 0, st>>>(part, ml, nseg, H, v_scale, o, lse);
  else
    sparse_combine<40><<<grid, kHeadDim, 0, st>>>(part, ml, nseg, H, v_scale, o, lse);
}

// Logit scale in base 2 and output scale of a descriptor (E4M3 caches fold
// their K scale into the first and V scale into the second).
float logit_c2(const hs2_attn_desc& d) {
  return d.sm_scale * kLog2e * (d.dtype == HS2_FP8_E4M3 ? d.k_scale : 1.f);
}
float out_scale(const hs2_attn_desc& d) { return d.dtype == HS2_FP8_E4M3 ? d.v_scale : 1.f; }

}  // namespace

hipError_t launch_sparse(const hs2_attn_desc& d, const void* q, const void* k, const void* v,
                         int64_t kv_stride, const int32_t* ctx_len, int cap,
                         const int32_t* top_idx, const int32_t* top_cnt, float* o, float* lse,
                         char* ws, hipStream_t st) {
  const SparseWs w = sparse_ws(d);
  float* part = reinterpret_cast<float*>(ws + w.part_off);
  float2* ml = reinterpret_cast<float2*>(ws + w.ml_off);
  const float c2 = logit_c2(d);
  int nseg;
  if (d.dtype != HS2_F32) {
    nseg = mfma_segments(d);
    const dim3 grid(nseg, d.batch * d.n_q);
    const auto* qq = static_cast<const uint16_t*>(q);
    if (d.dtype == HS2_FP8_E4M3)
      sparse_partial_bf16<true><<<grid, 64 * kSegWaves, 0, st>>>(
          qq, k, v, kv_stride, ctx_len, cap, top_idx, top_cnt, d.n_q, d.tile_q, d.k_top,
          d.window, d.n_heads, c2, part, ml, nseg);
    else
      sparse_partial_bf16<false><<<grid, 64 * kSegWaves, 0, st>>>(
          qq, k, v, kv_stride, ctx_len, cap, top_idx, top_cnt, d.n_q, d.tile_q, d.k_top,
          d.window, d.n_heads, c2, part, ml, nseg);
  } else {
    nseg = sparse_segments(d);
    sparse_partial_f32<<<dim3(nseg, d.batch * d.n_q), 256, 0, st>>>(
        static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
        kv_stride, ctx_len, cap, top_idx, top_cnt, d.n_q, d.tile_q, d.k_top, d.window,
        d.n_heads, c2, part, ml, nseg);
  }
  launch_combine(dim3(d.n_heads, d.batch * d.n_q), st, part, ml, nseg, d.n_heads, out_scale(d), o,
                 lse);
  return hipGetLastError();
}

hipError_t launch_decode_tail(const hs2_attn_desc& d, const void* q, const void* k, const void* v,
                              int64_t kv_stride, const int32_t* ctx_len, int cap,
                              const uint32_t* hist, const char* sel_ws, int32_t* top_idx,
                              int32_t* top_cnt, float* o, float* lse, char* ws, hipStream_t st) {
  const SparseWs w = sparse_ws(d);
  const SelectWs sw = select_ws(d, cap);
  float* part = reinterpret_cast<float*>(ws + w.part_off);
  float2* ml = reinterpret_cast<float2*>(ws + w.ml_off);
  const int nseg = mfma_segments(d);
  const dim3 grid(nseg, d.batch);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* cnt = reinterpret_cast<const uint32_t*>(sel_ws + sw.cnt_off);
  const auto* meta = reinterpret_cast<const uint32_t*>(sel_ws + sw.meta_off);
  const auto* list = reinterpret_cast<const uint2*>(sel_ws + sw.list_off);
  if (d.dtype == HS2_FP8_E4M3)
    decode_tail_bf16<true><<<grid, kTailThreads, 0, st>>>(
        qq, k, v, kv_stride, ctx_len, cap, d.k_top, d.window, d.n_heads, logit_c2(d), hist, cnt,
        meta, list, select_slices(cap), top_idx, top_cnt, part, ml, nseg);
  else
    decode_tail_bf16<false><<<grid, kTailThreads, 0, st>>>(
        qq, k, v, kv_stride, ctx_len, cap, d.k_top, d.window, d.n_heads, logit_c2(d), hist, cnt,
        meta, list, select_slices(cap), top_idx, top_cnt, part, ml, nseg);
  launch_combine(dim3(d.n_heads, d.batch), st, part, ml, nseg, d.n_heads, out_scale(d), o, lse);
  return hipGetLastError();
}

hipError_t launch_sparse_layers(const hs2_attn_desc& d, int n_layers, const void* q_layers,
                                const void* k, const void* v, int64_t kv_stride,
                                const int32_t* ctx_len, int cap, const int32_t* top_idx,
                                const int32_t* top_cnt, float* o_layers, float* lse_layers,
                                char* ws, hipStream_t st) {
  const int nseg = mfma_segments(d);
  const size_t rows = (size_t)n_layers * d.batch;
  float* part = reinterpret_cast<float*>(ws);
  float2* ml = reinterpret_cast<float2*>(
      ws + align_up(sizeof(float) * rows * nseg * d.n_heads * kHeadDim, 256));
  const dim3 grid(nseg, d.batch);
  const auto* qq = static_cast<const uint16_t*>(q_layers);
  if (d.dtype == HS2_FP8_E4M3)
    sparse_layers_bf16<true><<<grid, 64 * kSegWaves, 0, st>>>(
        qq, k, v, kv_stride, ctx_len, cap, top_idx, top_cnt, d.batch, d.k_top, d.window,
        d.n_heads, logit_c2(d), n_layers, part, ml, nseg);
  else
    sparse_layers_bf16<false><<<grid, 64 * kSegWaves, 0, st>>>(
        qq, k, v, kv_stride, ctx_len, cap, top_idx, top_cnt, d.batch, d.k_top, d.window,
        d.n_heads, logit_c2(d), n_layers, part, ml, nseg);
  launch_combine(dim3(d.n_heads, (int)rows), st, part, ml, nseg, d.n_heads, out_scale(d), o_layers,
                 lse_layers);
  return hipGetLastError();
}

}  // namespace hs2
