// Chunked prefill: full-layer scoring over query tiles and the tiles' sparse
// attention.
//
// HySparse2's full-attention layer yields the token selection that the
// following sparse layers reuse, and every sparse query also sees its 128
// most recent tokens ("HySparse2: How Xiaomi Split the Transformer to Fix
// Agent Prefill Costs", section "KV Reuse and Token-Level Sparse
// Selection").  For a block of new queries (chunked prefill) the importance of
// key j for a tile t of tile_q consecutive queries is the softmax probability
// summed over the tile's queries and all heads, each query normalised over
// its own causal range:
//   I_t[j] = sum_{i in t} sum_h 2^(x_ihj - L_ih),  j <= P_i,
// and the tile's queries share one top-k selection (pool [0, P_0 - window + 1)
// with P_0 the tile's first query) while each keeps its own window.
//
// One tiled MFMA core serves the three passes.  A wave owns one query (its
// heads padded to 32 rows); 16 waves (16 queries) share K blocks of 64 keys
// staged in LDS with a 272-byte row pitch (conflict-free 16-byte operand
// reads).  The logit tile uses eight v_mfma_f32_32x32x16_bf16 per 32 keys:
//   pf_stats:  K as the A operand: a lane owns one (query, head) row over 16
//              keys, so row max/sum stay in-lane; per key split, partial
//              (max, sum) per row.
//   pf_colsum: Q as the A operand: a lane owns one key over 16 rows; after
//              p = 2^(x - L) the column sum over the wave's rows is one more
//              MFMA against a vector of ones, with p split into a bf16 high
//              and low part so the sum keeps about fp32 accuracy; the 16
//              waves are added in a fixed order and written per
//              (16-query block, key).
//   pf_reduce: I_t[j] = sum of the tile's 16-query blocks, in order.
//   pf_sparse: 8 queries per workgroup; gathered keys (the tile's selection,
//              then the window band of the block), a statistics pass then a P.V pass on MFMA with V
//              transposed through LDS; exact normalisation, no rescaling.
#include "hs2_internal.h"

namespace hs2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

constexpr float kLn2 = 0.69314718055994531f;
constexpr int kBlk = 64;                        // keys per LDS stage
constexpr int kRowB = kHeadDim * 2 + 16;        // LDS bytes per K row
constexpr int kVtP = kBlk + 8;                  // bf16 per transposed-V row

__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  l = l * fast_exp2(m - mn) + l2 * fast_exp2(m2 - mn);
  m = mn;
}

// Q rows of one query as MFMA operand registers (lane: head r32, dims
// 16e + 8hh); heads >= H are zero.
__device__ __forceinline__ void load_q(const uint16_t* qrow, int H, int r32, int hh, bool live,
                                       bf16x8_t (&qr)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (live && r32 < H) x = *reinterpret_cast<const u32x4*>(qrow + r32 * kHeadDim + 16 * e + 8 * hh);
    qr[e] = as_bf16x8(x);
  }
}

// Stage 64 K rows (indices from `row_of`) into LDS; each thread moves 16 B.
template <typename RowOf>
__device__ __forceinline__ void stage_k(uint8_t* dst, const uint16_t* kb, RowOf row_of) {
  for (int e = threadIdx.x; e < kBlk * 16; e += blockDim.x) {
    const int r = e >> 4, c = e & 15;
    const u32x4 x = *reinterpret_cast<const u32x4*>(kb + (size_t)row_of(r) * kHeadDim + 8 * c);
    *reinterpret_cast<u32x4*>(dst + r * kRowB + 16 * c) = x;
  }
}

// Operand e of key row `key` in the staged block (dims 16e + 8hh).
__device__ __forceinline__ bf16x8_t k_opnd(const uint8_t* blk, int key, int e, int hh) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(blk + key * kRowB + 32 * e + 16 * hh));
}

// K blocks of the two scoring passes go through a ring of LDS slots filled by
// direct global-to-LDS loads (16 bytes a lane, no registers in between), so
// that the next blocks load while one is in the MFMAs.  A slot holds 64 rows
// of 256 bytes; the 16-byte chunks of row r are stored rotated by r % 16
// (chunk c at c ^ (r % 16)), which keeps the operand reads of 16 consecutive
// rows on distinct banks.  The compiler does not track these loads: a wave
// waits for its own with an explicit vmcnt, and a barrier then publishes the
// whole block.
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kRing = 3;                  // blocks in LDS: one in use, two loading
constexpr int kSlotB = kBlk * kHeadDim * 2;  // 16 KiB

// 64 rows by 16 waves of a 1024-thread workgroup: wave w moves rows
// 4w .. 4w+3, lane l the stored chunk l % 16 of row 4w + l / 16.
template <typename RowOf>
__device__ __forceinline__ void dma_k_block(uint8_t* slot, const uint16_t* kb, RowOf row_of) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = 4 * wave + (lane >> 4);
  const int c = (lane & 15) ^ (r & 15);
  __builtin_amdgcn_global_load_lds(kb + (size_t)row_of(r) * kHeadDim + 8 * c,
                                   (lds_void_t*)(slot + wave * 1024), 16, 0, 0);
}

__device__ __forceinline__ bf16x8_t k_opnd_ring(const uint8_t* slot, int key, int e, int hh) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(
      slot + key * (kHeadDim * 2) + 16 * ((2 * e + hh) ^ (key & 15))));
}

// Wait until this wave has at most `younger` (0 or 1) ring loads in flight and
// its LDS operations are done, then meet the other waves.
__device__ __forceinline__ void ring_barrier(bool younger) {
  if (younger) __builtin_amdgcn_s_waitcnt(1 | (7 << 4));  // vmcnt(1) lgkmcnt(0)
  else __builtin_amdgcn_s_waitcnt(0 | (7 << 4));          // vmcnt(0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

struct PfArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t kv_stride;
  const int32_t* ctx_len;
  int cap, n_q, H, tile_q, nsplit, split;
  float c2;
  float2* stats;   // [B][nsplit][n_q][32]
  float* colsum;   // [B][n_q/16][cap]
  float* lse_out;  // [B][n_q][H] or null
  // sparse
  const int32_t* top_idx;
  const int32_t* top_cnt;
  int k_top, window;
  float* o;        // [B][n_q][H][D]
  float* lse_sp;   // [B][n_q][H] or null
};

// ---------------------------------------------------------------------------
// Pass 1: partial (max, sum) per (query, head) row over one key split.
__global__ __launch_bounds__(1024) void pf_stats(PfArgs a) {
  const int rb = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  const int N = clamp_ctx(a.ctx_len, b, a.cap);
  const int i = rb * 16 + wave;             // this wave's query
  const int P = N - a.n_q + i;              // its position
  const int P_last = N - a.n_q + rb * 16 + 15;
  const int j0 = s * a.split;
  const int j1 = min(j0 + a.split, P_last + 1);
  float2* st = a.stats + (((size_t)b * a.nsplit + s) * a.n_q + i) * 32;
  if (P_last < 0 || j0 >= j1) {
    if (hh == 0) st[r32] = make_float2(-INFINITY, 0.f);
    return;
  }
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing * kSlotB];
  bf16x8_t qr[8];
  load_q(a.q + ((size_t)b * a.n_q + i) * a.H * kHeadDim, a.H, r32, hh, P >= 0, qr);
  const uint16_t* kb = a.k + (size_t)b * a.kv_stride;
  const int nblk = (j1 - j0 + kBlk - 1) / kBlk;
  auto rows_of = [&](int bi) { return [=](int r) { return min(j0 + bi * kBlk + r, j1 - 1); }; };
  // Q is in registers before the ring starts, so that no later wait for it
  // has to cover the ring loads.
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0)
  dma_k_block(ring, kb, rows_of(0));
  if (nblk > 1) dma_k_block(ring + kSlotB, kb, rows_of(1));
  float m = -INFINITY, l = 0.f;
  for (int bi = 0; bi < nblk; ++bi) {
    // Block bi has landed for every wave; the slot of block bi-1 is free.
    ring_barrier(bi + 1 < nblk);
    if (bi + 2 < nblk) dma_k_block(ring + ((bi + 2) % kRing) * kSlotB, kb, rows_of(bi + 2));
    const uint8_t* kblk = ring + (bi % kRing) * kSlotB;
    const int kb0 = j0 + bi * kBlk;
    if (P < kb0) continue;  // the whole block is in this query's future
    // Every key of the block is inside this query's range and the split:
    // no masks, and the scale folds into one fma per logit (c2 > 0).
    const bool full = kb0 + kBlk <= j1 && kb0 + kBlk - 1 <= P;
    f32x16_t accs[2] = {{}, {}};
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        accs[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_opnd_ring(kblk, 32 * mt + r32, e, hh), qr[e], accs[mt], 0, 0, 0);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const f32x16_t& acc = accs[mt];
      // acc[r]: row (query i, head r32), key kb0 + 32mt + 8(r/4) + 4hh + r%4
      // The running reference m moves only when a logit exceeds it by more
      // than 64 binades: the block's terms are summed against the current m
      // (each at most 2^64, so the sum stays finite and keeps fp32 relative
      // precision), and only a sum above 2^64 (or a first block) takes the
      // block maximum and rescales.  This saves the 16 max operations per
      // half on almost every block.
      float lazy = 0.f;
      if (full && m != -INFINITY) {
#pragma unroll
        for (int r = 0; r < 16; ++r) lazy += fast_exp2(fmaf(acc[r], a.c2, -m));
      }
      if (full && m != -INFINITY && lazy <= 0x1p64f) {
        l += lazy;
      } else if (full) {
        float bm = acc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) bm = fmaxf(bm, acc[r]);
        const float mn = fmaxf(m, bm * a.c2);
        float sum = l * fast_exp2(m - mn);
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += fast_exp2(fmaf(acc[r], a.c2, -mn));
        l = sum;
        m = mn;
      } else {
        float x[16];
        float bm = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kb0 + 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
          x[r] = (j < j1 && j <= P) ? acc[r] * a.c2 : -INFINITY;
          bm = fmaxf(bm, x[r]);
        }
        const float mn = fmaxf(m, bm);
        const float mref = (mn == -INFINITY) ? 0.f : mn;
        float sum = l * fast_exp2(m - mref);
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += fast_exp2(x[r] - mref);
        l = sum;
        m = mn;
      }
    }
  }
  merge_ml(m, l, __shfl_xor(m, 32), __shfl_xor(l, 32));
  if (hh == 0) st[r32] = make_float2(m, l);
}

// Fold the split statistics of the workgroup's 16 x 32 rows into L (base 2;
// +inf for padded heads and empty rows so that 2^(x - L) = 0).
__device__ void fold_rows(const PfArgs& a, int b, int rb, int N, float* s_L, bool write_lse) {
  const int t = threadIdx.x;  // threads t < 512: one (query, head) row each
  if (t < 16 * 32) {
    const int qi = t >> 5, h = t & 31, i = rb * 16 + qi;
    const int P_last = N - a.n_q + rb * 16 + 15;
    const int ns = P_last < 0 ? 0 : min(a.nsplit, (P_last + a.split) / a.split);
    float m = -INFINITY, l = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float2 v = a.stats[(((size_t)b * a.nsplit + s) * a.n_q + i) * 32 + h];
      merge_ml(m, l, v.x, v.y);
    }
    const bool live = h < a.H && l > 0.f;
    s_L[t] = live ? m + log2f(l) : INFINITY;
    if (write_lse && a.lse_out != nullptr && h < a.H)
      a.lse_out[((size_t)b * a.n_q + i) * a.H + h] = live ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
  __syncthreads();
}

// Pass 2: per (16-query block, key) column sums of p over the block's rows.
__global__ __launch_bounds__(1024) void pf_colsum(PfArgs a) {
  const int rb = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  const int N = clamp_ctx(a.ctx_len, b, a.cap);
  const int i = rb * 16 + wave;
  const int P = N - a.n_q + i;
  const int P_last = N - a.n_q + rb * 16 + 15;
  const int j0 = s * a.split;
  const int j1 = min(j0 + a.split, P_last + 1);
  if (P_last < 0 || j0 >= j1) {
    // A block entirely before the cache start sees no key: log-sum-exp -inf.
    if (P_last < 0 && s == 0 && a.lse_out != nullptr && hh == 0 && r32 < a.H)
      a.lse_out[((size_t)b * a.n_q + i) * a.H + r32] = -INFINITY;
    return;
  }
  // One LDS object: with several, the compiler tracks the ring loads per
  // object and waits for all of them before any read of the ring.
  __shared__ struct __attribute__((aligned(16))) {
    uint8_t ring[kRing * kSlotB];
    float s_L[16 * 32];
    float s_cs[2][16][kBlk];
  } sm;
  uint8_t* ring = sm.ring;
  float* s_L = sm.s_L;
  auto& s_cs = sm.s_cs;
  fold_rows(a, b, rb, N, s_L, s == 0);
  bf16x8_t qr[8];
  load_q(a.q + ((size_t)b * a.n_q + i) * a.H * kHeadDim, a.H, r32, hh, P >= 0, qr);
  float L[16];  // rows (heads) 8(r/4) + 4hh + r%4 of this wave's query
#pragma unroll
  for (int r = 0; r < 16; ++r) L[r] = s_L[wave * 32 + 8 * (r >> 2) + 4 * hh + (r & 3)];
  const uint16_t* kb = a.k + (size_t)b * a.kv_stride;
  float* out = a.colsum + ((size_t)b * (a.n_q / 16) + rb) * a.cap;
  const int nblk = (j1 - j0 + kBlk - 1) / kBlk;
  auto rows_of = [&](int bi) { return [=](int r) { return min(j0 + bi * kBlk + r, j1 - 1); }; };
  // Q is in registers before the ring starts, so that no later wait for it
  // has to cover the ring loads.
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0)
  dma_k_block(ring, kb, rows_of(0));
  if (nblk > 1) dma_k_block(ring + kSlotB, kb, rows_of(1));
  auto block_sum = [&](int bj) {
    if (threadIdx.x < kBlk) {
      const int j = j0 + bj * kBlk + threadIdx.x;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < 16; ++w) sum += s_cs[bj & 1][w][threadIdx.x];
      if (j < j1) out[j] = sum;
    }
  };
  for (int bi = 0; bi < nblk; ++bi) {
    ring_barrier(bi + 1 < nblk);
    if (bi + 2 < nblk) dma_k_block(ring + ((bi + 2) % kRing) * kSlotB, kb, rows_of(bi + 2));
    if (bi > 0) block_sum(bi - 1);
    const uint8_t* kblk = ring + (bi % kRing) * kSlotB;
    const int kb0 = j0 + bi * kBlk;
    const bool full = kb0 + kBlk <= j1 && kb0 + kBlk - 1 <= P;
    f32x16_t accs[2] = {{}, {}};
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        accs[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qr[e], k_opnd_ring(kblk, 32 * mt + r32, e, hh), accs[mt], 0, 0, 0);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int j = kb0 + 32 * mt + r32;  // this lane's key
      const f32x16_t& acc = accs[mt];
      // acc[r]: row (query i, head 8(r/4) + 4hh + r%4), key j.  The sum over
      // the query's 32 head rows: 16 in this lane, 16 in lane ^ 32.  Padded
      // heads have L = +inf, so their p is 0.
      float cs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) cs += fast_exp2(fmaf(acc[r], a.c2, -L[r]));
      if (!full && !(j < j1 && j <= P)) cs = 0.f;
      cs += __shfl_xor(cs, 32);
      if (hh == 0) s_cs[bi & 1][wave][32 * mt + r32] = cs;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  block_sum(nblk - 1);
}

// ---------------------------------------------------------------------------
// The full layer's own output, o_full[i][h] = sum_j p_ihj v_j over each
// query's causal range, exactly normalised with the statistics of pf_stats
// (p = 2^(x - L), no running rescale).  A 512-thread workgroup owns 8
// consecutive queries (a wave each) over all their keys, so no partial
// outputs need merging, and a wave has 256 registers for O (four 32x32
// fp32 tiles), Q and the logit tile.  K and V blocks of 64 keys come through
// a ring of LDS slots like the scoring passes (rotated chunk layout); after
// the block's barrier the workgroup transposes V into vt (wave w: dims
// 16w .. 16w + 15, lane: key) and a second barrier publishes it.  K is the
// A operand, so a lane holds one head over 16 keys, which is the B layout of
// P^T: O^T += V^T P^T with p as a bf16 high and low part (residual below
// 2^-17 of p).
constexpr int kOutWaves = 8;

// 64 rows by the 8 waves of a 512-thread workgroup: wave w moves rows
// 8w .. 8w + 7 in two loads, lane l the stored chunk l % 16 of a row.
template <typename RowOf>
__device__ __forceinline__ void dma_block_w8(uint8_t* slot, const uint16_t* base, RowOf row_of) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int r = 8 * wave + 4 * k + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    __builtin_amdgcn_global_load_lds(base + (size_t)row_of(r) * kHeadDim + 8 * c,
                                     (lds_void_t*)(slot + wave * 2048 + k * 1024), 16, 0, 0);
  }
}

__global__ __launch_bounds__(512) void pf_out(PfArgs a, float* __restrict__ o_full) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  const int N = clamp_ctx(a.ctx_len, b, a.cap);
  const int i = blockIdx.x * kOutWaves + wave;
  const int P = N - a.n_q + i;
  const int P_last = N - a.n_q + blockIdx.x * kOutWaves + kOutWaves - 1;
  f32x16_t o[4] = {{}, {}, {}, {}};  // O^T: dims 32t + 8(r/4) + 4hh + r%4, head r32
  if (P_last >= 0) {
    __shared__ struct __attribute__((aligned(16))) {
      uint8_t ring[kRing][2][kSlotB];  // [slot][K, V]
      uint16_t vt[kHeadDim][kVtP];
      float s_L[16 * 32];
    } sm;
    // Statistics of the enclosing 16-query block; this workgroup is one half.
    fold_rows(a, b, blockIdx.x >> 1, N, sm.s_L, false);
    bf16x8_t qr[8];
    load_q(a.q + ((size_t)b * a.n_q + i) * a.H * kHeadDim, a.H, r32, hh, P >= 0, qr);
    // +inf for padded heads and queries that see no key, so that p = 0.
    const float Lh = sm.s_L[((blockIdx.x & 1) * kOutWaves + wave) * 32 + r32];
    const int j1 = P_last + 1;
    const uint16_t* kb = a.k + (size_t)b * a.kv_stride;
    const uint16_t* vb = a.v + (size_t)b * a.kv_stride;
    const int nblk = (j1 + kBlk - 1) / kBlk;
    auto issue = [&](int bi) {
      auto rows = [=](int r) { return min(bi * kBlk + r, j1 - 1); };
      dma_block_w8(sm.ring[bi % kRing][0], kb, rows);
      dma_block_w8(sm.ring[bi % kRing][1], vb, rows);
    };
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4));  // vmcnt(0) lgkmcnt(0): Q
    issue(0);
    if (nblk > 1) issue(1);
    for (int bi = 0; bi < nblk; ++bi) {
      // Block bi (four loads per wave) has landed for every wave once the
      // younger block's four are all that is in flight; the slot of block
      // bi - 1 and vt are free after the barrier.
      if (bi + 1 < nblk)
        __builtin_amdgcn_s_waitcnt(4 | (7 << 4));  // vmcnt(4) lgkmcnt(0)
      else
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      if (bi + 2 < nblk) issue(bi + 2);
      const uint8_t* ks = sm.ring[bi % kRing][0];
      const uint8_t* vs = sm.ring[bi % kRing][1];
      // Key `lane` goes to column vpos (bits 2 and 3 swapped), so that the
      // eight keys of one MFMA operand sit side by side (see below).
      const int vpos = (lane & ~12) | ((lane & 4) << 1) | ((lane & 8) >> 1);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        // Chunk c = 2w + cc (dims 8c .. 8c + 7) of key row `lane`, stored at
        // chunk position c ^ (lane % 16).
        const int c = 2 * wave + cc;
        const u32x4 x = *reinterpret_cast<const u32x4*>(vs + lane * (kHeadDim * 2) +
                                                         16 * (c ^ (lane & 15)));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sm.vt[8 * c + 2 * e][vpos] = (uint16_t)(x[e] & 0xFFFFu);
          sm.vt[8 * c + 2 * e + 1][vpos] = (uint16_t)(x[e] >> 16);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      const int kb0 = bi * kBlk;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x16_t acc = {};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_opnd_ring(ks, 32 * mt + r32, e, hh),
                                                        qr[e], acc, 0, 0, 0);
        // acc[r]: head r32, key kb0 + 32mt + 8(r/4) + 4hh + r%4.  The MFMA
        // k index 8hh + jj of step sp stands for the lane's p[8sp + jj], key
        // 32mt + 16sp + 8(jj/4) + 4hh + jj%4, in A (V^T) and B (P^T) alike;
        // that key's vt column is 32mt + 16sp + 8hh + jj.
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          u32x4 phi, plo;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            float pp[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int r = 8 * sp + 2 * jj + u;
              const int j = kb0 + 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
              pp[u] = (j <= P) ? fast_exp2(fmaf(acc[r], a.c2, -Lh)) : 0.f;
            }
            const uint16_t h0 = f32_to_bf16_rne(pp[0]), h1 = f32_to_bf16_rne(pp[1]);
            const uint16_t l0 = f32_to_bf16_rne(pp[0] - bf16_to_f32(h0));
            const uint16_t l1 = f32_to_bf16_rne(pp[1] - bf16_to_f32(h1));
            phi[jj] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            plo[jj] = (uint32_t)l0 | ((uint32_t)l1 << 16);
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const u32x4 av =
                *reinterpret_cast<const u32x4*>(&sm.vt[32 * t + r32][32 * mt + 16 * sp + 8 * hh]);
            o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(phi), o[t],
                                                           0, 0, 0);
            o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(plo), o[t],
                                                           0, 0, 0);
          }
        }
      }
    }
  }
  // Queries before the cache start and padded heads have p = 0, so O = 0.
  if (r32 < a.H) {
    float* orow = o_full + (((size_t)b * a.n_q + i) * a.H + r32) * kHeadDim;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(orow + 32 * t + 8 * g + 4 * hh) =
            f32x4{o[t][4 * g], o[t][4 * g + 1], o[t][4 * g + 2], o[t][4 * g + 3]};
  }
}

// I_t[j] = sum over the tile's 16-query blocks (in order) of their column
// sums; a block contributes only to keys inside its causal range.  Optionally
// histograms the pool keys for the selector.
template <bool kHist>
__global__ __launch_bounds__(256) void pf_reduce(PfArgs a, float* scores, uint32_t* hist) {
  const int t = blockIdx.y, b = blockIdx.z;
  const int tiles = a.n_q / a.tile_q;
  const int per = a.tile_q / 16;
  const int N = clamp_ctx(a.ctx_len, b, a.cap);
  const int P0 = N - a.n_q + t * a.tile_q;
  const int pe = max(0, P0 - a.window + 1);
  __shared__ uint32_t s_hist[kHist ? kSelBins : 1];
  if (kHist) {
    for (int e = threadIdx.x; e < kSelBins; e += blockDim.x) s_hist[e] = 0u;
    __syncthreads();
  }
  const int j0 = blockIdx.x * 4096;
  for (int j = j0 + threadIdx.x; j < min(N, j0 + 4096); j += blockDim.x) {
    float sum = 0.f;
    for (int r = 0; r < per; ++r) {
      const int rb = t * per + r;
      const int P_last = N - a.n_q + rb * 16 + 15;
      if (j <= P_last) sum += a.colsum[((size_t)b * (a.n_q / 16) + rb) * a.cap + j];
    }
    scores[((size_t)b * tiles + t) * a.cap + j] = sum;
    if (kHist && j < pe) atomicAdd(&s_hist[order_key(sum) >> 20], 1u);
  }
  if (kHist) {
    __syncthreads();
    uint32_t* gh = hist + ((size_t)b * tiles + t) * kHistRow;
    for (int e = threadIdx.x; e < kSelBins; e += blockDim.x)
      if (s_hist[e] != 0u) atomicAdd(&gh[e], s_hist[e]);
  }
}

__global__ __launch_bounds__(256) void pf_hist_init(uint32_t* hist) {
  for (int e = threadIdx.x; e < kHistRow; e += blockDim.x) hist[(size_t)blockIdx.x * kHistRow + e] = 0u;
}

// ---------------------------------------------------------------------------
// Sparse attention of an 8-query block over its tile's selection plus the
// block's window band: S_i = T_t ++ [max(0, P_i - W + 1), P_i].
constexpr int kSpWaves = 8;  // queries per workgroup of the sparse pass

__global__ __launch_bounds__(64 * kSpWaves) void pf_sparse(PfArgs a) {
  const int rb = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  const int tiles = a.n_q / a.tile_q;
  const int N = clamp_ctx(a.ctx_len, b, a.cap);
  const int i = rb * kSpWaves + wave;
  const int P = N - a.n_q + i;
  const int t = (rb * kSpWaves) / a.tile_q;
  const int P_first = N - a.n_q + rb * kSpWaves, P_last = P_first + kSpWaves - 1;
  int cnt = 0;
  if (P_last >= 0) {
    cnt = a.top_cnt[b * tiles + t];
    cnt = cnt < 0 ? 0 : (cnt > a.k_top ? a.k_top : cnt);
  }
  // Band: keys [band_lo, P_last] (the union of the block's windows).
  const int band_lo = max(0, P_first - a.window + 1);
  const int band = P_last >= 0 ? P_last - band_lo + 1 : 0;
  const int total = cnt + band;
  const int32_t* top_row = a.top_idx + (size_t)(b * tiles + t) * a.k_top;
  auto key_of = [&](int p) -> int {
    int idx = p < cnt ? top_row[p] : band_lo + (p - cnt);
    return idx < 0 ? 0 : (idx >= N ? N - 1 : idx);
  };
  // Key at list position p is visible to query position P: selected keys
  // always (they precede every window of the tile), band keys inside the
  // query's own window.
  auto visible = [&](int p, int key) -> bool {
    if (p >= total) return false;
    if (p < cnt) return true;
    return key <= P && key > P - a.window;
  };

  __shared__ __attribute__((aligned(16))) uint8_t kblk[kBlk * kRowB];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kHeadDim][kVtP];
  __shared__ int s_key[kBlk];
  bf16x8_t qr[8];
  load_q(a.q + ((size_t)b * a.n_q + i) * a.H * kHeadDim, a.H, r32, hh, P >= 0, qr);
  const uint16_t* kb = a.k + (size_t)b * a.kv_stride;
  const uint16_t* vb = a.v + (size_t)b * a.kv_stride;

  // Pass A: row statistics over the list.
  float m = -INFINITY, l = 0.f;
  for (int p0 = 0; p0 < total; p0 += kBlk) {
    __syncthreads();
    if (threadIdx.x < kBlk) s_key[threadIdx.x] = key_of(min(p0 + (int)threadIdx.x, total - 1));
    __syncthreads();
    stage_k(kblk, kb, [&](int r) { return s_key[r]; });
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16_t acc = {};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_opnd(kblk, 32 * mt + r32, e, hh), qr[e], acc, 0, 0, 0);
      float x[16];
      float bm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kp = 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
        x[r] = (P >= 0 && visible(p0 + kp, s_key[kp])) ? acc[r] * a.c2 : -INFINITY;
        bm = fmaxf(bm, x[r]);
      }
      const float mn = fmaxf(m, bm);
      const float mref = (mn == -INFINITY) ? 0.f : mn;
      float sum = l * fast_exp2(m - mref);
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += fast_exp2(x[r] - mref);
      l = sum;
      m = mn;
    }
  }
  merge_ml(m, l, __shfl_xor(m, 32), __shfl_xor(l, 32));
  const float Lrow = (l > 0.f) ? m + log2f(l) : INFINITY;  // this lane's row (head r32)

  // Pass B: O = sum_j 2^(x - L) v_j.
  f32x16_t o[4] = {{}, {}, {}, {}};
  for (int p0 = 0; p0 < total; p0 += kBlk) {
    __syncthreads();
    if (threadIdx.x < kBlk) s_key[threadIdx.x] = key_of(min(p0 + (int)threadIdx.x, total - 1));
    __syncthreads();
    stage_k(kblk, kb, [&](int r) { return s_key[r]; });
    // V block transposed: vt[d][key].
    for (int e = threadIdx.x; e < kBlk * 16; e += blockDim.x) {
      const int r = e >> 4, c = e & 15;
      const u32x4 x = *reinterpret_cast<const u32x4*>(vb + (size_t)s_key[r] * kHeadDim + 8 * c);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        vt[8 * c + 2 * u][r] = (uint16_t)(x[u] & 0xFFFFu);
        vt[8 * c + 2 * u + 1][r] = (uint16_t)(x[u] >> 16);
      }
    }
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16_t acc = {};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_opnd(kblk, 32 * mt + r32, e, hh), qr[e], acc, 0, 0, 0);
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kp = 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
        pr[r] = (P >= 0 && visible(p0 + kp, s_key[kp])) ? fast_exp2(acc[r] * a.c2 - Lrow) : 0.f;
      }
      // P V: A = p (row = head r32, keys in register order), B = V^T rows.
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 hi, lo;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float p0v = pr[8 * ks + 2 * u], p1v = pr[8 * ks + 2 * u + 1];
          const uint16_t h0 = f32_to_bf16_rne(p0v), h1 = f32_to_bf16_rne(p1v);
          hi[u] = (uint32_t)h0 | ((uint32_t)h1 << 16);
          lo[u] = (uint32_t)f32_to_bf16_rne(p0v - bf16_to_f32(h0)) |
                  ((uint32_t)f32_to_bf16_rne(p1v - bf16_to_f32(h1)) << 16);
        }
        const int kbase = 32 * mt + 16 * ks + 4 * hh;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const uint16_t* row = &vt[32 * dt + r32][0];
          const uint2 a4 = *reinterpret_cast<const uint2*>(row + kbase);
          const uint2 b4 = *reinterpret_cast<const uint2*>(row + kbase + 8);
          const u32x4 bv = {a4.x, a4.y, b4.x, b4.y};
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(hi), as_bf16x8(bv), o[dt], 0, 0, 0);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lo), as_bf16x8(bv), o[dt], 0, 0, 0);
        }
      }
    }
  }
  // o[dt][r]: row head 8(r/4) + 4hh + r%4, dim 32dt + r32 (already normalised;
  // a query before the cache start has l = 0, p = 0 and writes zeros).
  {
    float* orow = a.o + ((size_t)b * a.n_q + i) * a.H * kHeadDim;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int h = 8 * (r >> 2) + 4 * hh + (r & 3);
      if (h < a.H)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) orow[(size_t)h * kHeadDim + 32 * dt + r32] = o[dt][r];
    }
    if (a.lse_sp != nullptr && hh == 0 && r32 < a.H)
      a.lse_sp[((size_t)b * a.n_q + i) * a.H + r32] = (l > 0.f) ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

}  // namespace

// Workspace of the prefill scoring (inside the scoring region):
//   stats  float2 [B][nsplit][n_q][32]
//   colsum float  [B][n_q/16][cap]
//   hist   uint32 [B][tiles][kHistRow]
hipError_t launch_prefill_scores(const hs2_attn_desc& d, const void* q, const void* k,
                                 int64_t kv_stride, const int32_t* ctx_len, int cap,
                                 float* scores, float* lse, char* ws, bool with_hist,
                                 hipStream_t st) {
  const PrefillWs w = prefill_ws(d, cap);
  PfArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.kv_stride = kv_stride;
  a.ctx_len = ctx_len;
  a.cap = cap;
  a.n_q = d.n_q;
  a.H = d.n_heads;
  a.tile_q = d.tile_q;
  a.split = kPfSplit;
  a.nsplit = (cap + kPfSplit - 1) / kPfSplit;
  a.c2 = d.sm_scale * 1.4426950408889634f;
  a.stats = reinterpret_cast<float2*>(ws + w.stats_off);
  a.colsum = reinterpret_cast<float*>(ws + w.colsum_off);
  a.lse_out = lse;
  a.window = d.window;
  const dim3 g(d.n_q / 16, a.nsplit, d.batch);
  pf_stats<<<g, 1024, 0, st>>>(a);
  pf_colsum<<<g, 1024, 0, st>>>(a);
  const int tiles = d.n_q / d.tile_q;
  const dim3 gr((cap + 4095) / 4096, tiles, d.batch);
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + w.hist_off);
  if (with_hist) {
    pf_hist_init<<<d.batch * tiles, 256, 0, st>>>(hist);
    pf_reduce<true><<<gr, 256, 0, st>>>(a, scores, hist);
  } else {
    pf_reduce<false><<<gr, 256, 0, st>>>(a, scores, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_out(const hs2_attn_desc& d, const void* q, const void* k,
                              const void* v, int64_t kv_stride, const int32_t* ctx_len, int cap,
                              float* o_full, char* ws, hipStream_t st) {
  const PrefillWs w = prefill_ws(d, cap);
  PfArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.kv_stride = kv_stride;
  a.ctx_len = ctx_len;
  a.cap = cap;
  a.n_q = d.n_q;
  a.H = d.n_heads;
  a.tile_q = d.tile_q;
  a.split = kPfSplit;
  a.nsplit = (cap + kPfSplit - 1) / kPfSplit;
  a.c2 = d.sm_scale * 1.4426950408889634f;
  a.stats = reinterpret_cast<float2*>(ws + w.stats_off);
  pf_out<<<dim3(d.n_q / kOutWaves, d.batch), 512, 0, st>>>(a, o_full);
  return hipGetLastError();
}

hipError_t launch_prefill_sparse(const hs2_attn_desc& d, const void* q, const void* k,
                                 const void* v, int64_t kv_stride, const int32_t* ctx_len,
                                 int cap, const int32_t* top_idx, const int32_t* top_cnt,
                                 float* o, float* lse, hipStream_t st) {
  PfArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.kv_stride = kv_stride;
  a.ctx_len = ctx_len;
  a.cap = cap;
  a.n_q = d.n_q;
  a.H = d.n_heads;
  a.tile_q = d.tile_q;
  a.c2 = d.sm_scale * 1.4426950408889634f;
  a.top_idx = top_idx;
  a.top_cnt = top_cnt;
  a.k_top = d.k_top;
  a.window = d.window;
  a.o = o;
  a.lse_sp = lse;
  pf_sparse<<<dim3(d.n_q / kSpWaves, d.batch), 64 * kSpWaves, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace hs2
