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
// One tiled MFMA core serves the scoring passes.  A workgroup owns a block
// of 16 queries; its 8 waves take two queries each (heads padded to 32
// rows) and share K blocks of 64 keys staged in LDS by direct-to-LDS loads
// (rows of 256 bytes, 16-byte chunks XOR-swizzled by row, so that operand
// reads are conflict-free).  The logit tile uses eight
// v_mfma_f32_32x32x16_bf16 per 32 keys and query, and each K operand read
// feeds the MFMAs of both queries:
//   pf_stats:  K as the A operand: a lane owns one (query, head) row over 16
//              keys, so row max/sum stay in-lane; per key split, partial
//              (max, sum) per row.
//   pf_colsum: Q as the A operand: a lane owns one key over 16 rows; after
//              p = 2^(x - L) the column sum over the wave's two queries is
//              an fp32 sum in the lane plus one add across the two lane
//              halves; the 8 waves are added in a fixed order, kept in LDS
//              for the split and written per (16-query block, key).
//   pf_reduce: I_t[j] = sum of the tile's 16-query blocks, in order.
//   pf_sparse: 8 queries per workgroup; gathered keys (the tile's selection,
//              then the window band of the block), a statistics pass then a P.V pass on MFMA with V
//              transposed through LDS; exact normalisation, no rescaling.
#include <type_traits>

#include "hs2_internal.h"

namespace hs2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

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

// Stage 64 K rows (indices from `row_of`) into LDS as bf16; each thread
// moves 16 B of a row (E4M3 rows: 16 bytes, widened to 32 B of bf16).
template <bool kFp8, typename RowOf>
__device__ __forceinline__ void stage_k(uint8_t* dst, const void* kb, RowOf row_of) {
  if constexpr (kFp8) {
    const uint8_t* k8 = static_cast<const uint8_t*>(kb);
    for (int e = threadIdx.x; e < kBlk * 8; e += blockDim.x) {
      const int r = e >> 3, c = e & 7;
      const u32x4 x = *reinterpret_cast<const u32x4*>(k8 + (size_t)row_of(r) * kHeadDim + 16 * c);
      *reinterpret_cast<u32x4*>(dst + r * kRowB + 32 * c) = e4m3x8_to_bf16x8(x[0], x[1]);
      *reinterpret_cast<u32x4*>(dst + r * kRowB + 32 * c + 16) = e4m3x8_to_bf16x8(x[2], x[3]);
    }
  } else {
    const uint16_t* k16 = static_cast<const uint16_t*>(kb);
    for (int e = threadIdx.x; e < kBlk * 16; e += blockDim.x) {
      const int r = e >> 4, c = e & 15;
      const u32x4 x = *reinterpret_cast<const u32x4*>(k16 + (size_t)row_of(r) * kHeadDim + 8 * c);
      *reinterpret_cast<u32x4*>(dst + r * kRowB + 16 * c) = x;
    }
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
constexpr int kRing = 3;                  // pf_out: blocks in LDS, one in use, two loading
constexpr int kSlotB = kBlk * kHeadDim * 2;  // 16 KiB

__device__ __forceinline__ bf16x8_t k_opnd_ring(const uint8_t* slot, int key, int e, int hh) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(
      slot + key * (kHeadDim * 2) + 16 * ((2 * e + hh) ^ (key & 15))));
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
  float v_scale;   // scale of the V cache (E4M3), else 1
};

// ---------------------------------------------------------------------------
// The two scoring passes run 8 waves of two consecutive queries each (a
// workgroup owns a 16-query block): every K operand read from LDS feeds the
// MFMAs of both queries, which halves the LDS traffic per FLOP, and the
// exponentials of one 32-key half are issued between the MFMAs of the next.
constexpr int kPfWaves = 8;
constexpr int kPfRing = 3;  // K blocks in LDS: the one in use and two loading

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

// E4M3 caches (one byte per element, 128-byte rows): a block of 64 rows comes
// through registers instead, thread t of the 512 holding bytes 16(t % 8) ..
// +15 of row t / 8, and is written widened to bf16 (exact: every E4M3 value
// is a bf16 value) into the same slot layout as a bf16 block, so that the
// MFMA code reads both alike.
template <typename RowOf>
__device__ __forceinline__ u32x4 load_block_e4m3(const uint8_t* base, RowOf row_of) {
  const int r = threadIdx.x >> 3, c = threadIdx.x & 7;
  return *reinterpret_cast<const u32x4*>(base + (size_t)row_of(r) * kHeadDim + 16 * c);
}

__device__ __forceinline__ void store_block_e4m3(uint8_t* slot, u32x4 x) {
  const int r = threadIdx.x >> 3, c = threadIdx.x & 7;
  uint8_t* row = slot + r * (kHeadDim * 2);
  *reinterpret_cast<u32x4*>(row + 16 * ((2 * c) ^ (r & 15))) = e4m3x8_to_bf16x8(x[0], x[1]);
  *reinterpret_cast<u32x4*>(row + 16 * ((2 * c + 1) ^ (r & 15))) = e4m3x8_to_bf16x8(x[2], x[3]);
}

// Wait until this wave's ring loads of the current block have landed (the
// younger block's two may still be in flight) and its LDS operations are
// done, then meet the other waves.  No other global memory operation is
// outstanding in the loops, so the count covers ring loads only.
__device__ __forceinline__ void ring_barrier_w8(bool younger) {
  if (younger) __builtin_amdgcn_s_waitcnt(2 | (7 << 4));  // vmcnt(2) lgkmcnt(0)
  else __builtin_amdgcn_s_waitcnt(0 | (7 << 4));          // vmcnt(0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Per-lane addresses of the lane's eight K operands (steps e) in the first
// half of a ring slot, as k_opnd_ring computes them for key r32; the second
// half is 32 rows further.  Formed before the MFMA section (a scheduling
// barrier keeps their arithmetic out of it).
__device__ __forceinline__ void k_opnd_ptrs(const uint8_t* slot, int r32, int hh,
                                            const uint8_t* (&kp)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) kp[e] = slot + r32 * (kHeadDim * 2) + 16 * ((2 * e + hh) ^ (r32 & 15));
  __builtin_amdgcn_sched_barrier(0);
}

// The logits of one 32-key half (mt) of the K block in a ring slot for the
// wave's two queries (fp32, unscaled): with K as the A operand (kKA) a lane
// holds (query, head r32) over 16 keys, with Q as the A operand one key over
// 16 heads.  `valu(e)` is issued between the MFMAs: the exponentials of the
// previous half, which then overlap this half's MFMAs.  Without that the
// per-block workgroup barrier keeps the waves of a SIMD in one phase, all on
// MFMA and then all on exponentials, and the two pipelines take turns.
template <bool kKA, typename V>
__device__ __forceinline__ void half_logits(const uint8_t* const (&kp)[8], int mt,
                                            const bf16x8_t (&qa)[8], const bf16x8_t (&qb)[8],
                                            f32x16_t (&acc)[2], V valu) {
  acc[0] = f32x16_t{};
  acc[1] = f32x16_t{};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bf16x8_t kop =
        as_bf16x8(*reinterpret_cast<const u32x4*>(kp[e] + mt * 32 * (kHeadDim * 2)));
    if (kKA) {
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qa[e], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qb[e], acc[1], 0, 0, 0);
    } else {
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[e], kop, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qb[e], kop, acc[1], 0, 0, 0);
    }
    valu(e);
  }
  // Per step: the next step's K operand read, then each MFMA followed by six
  // VALU operations (fma, exponential and add for two terms), about as long
  // as the MFMA.  Two MFMAs in a row would stall the wave at the second
  // (the matrix unit is busy), and its exponentials with it.
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e < 7) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);
  }
}

// Pass 1: partial (max, sum) per (query, head) row over one key split.
template <bool kFp8>
__global__ __launch_bounds__(64 * kPfWaves) void pf_stats(PfArgs a) {
  const int rb = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  const int N = clamp_ctx(a.ctx_len, b, a.cap);
  const int i0 = rb * 16 + 2 * wave;        // this wave's queries i0, i0 + 1
  const int P0 = N - a.n_q + i0;
  const int P_last = N - a.n_q + rb * 16 + 15;
  const int j0 = s * a.split;
  const int j1 = min(j0 + a.split, P_last + 1);
  float2* st = a.stats + (((size_t)b * a.nsplit + s) * a.n_q + i0) * 32;  // two rows of 32
  if (P_last < 0 || j0 >= j1) {
    if (hh == 0) {
      st[r32] = make_float2(-INFINITY, 0.f);
      st[32 + r32] = make_float2(-INFINITY, 0.f);
    }
    return;
  }
  __shared__ __attribute__((aligned(16))) uint8_t ring[kPfRing * kSlotB];
  bf16x8_t qa[8], qb[8];
  const uint16_t* qrow = a.q + ((size_t)b * a.n_q + i0) * a.H * kHeadDim;
  load_q(qrow, a.H, r32, hh, P0 >= 0, qa);
  load_q(qrow + a.H * kHeadDim, a.H, r32, hh, P0 + 1 >= 0, qb);
  const uint16_t* kb = a.k + (size_t)b * a.kv_stride;
  const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(a.k) + (size_t)b * a.kv_stride;
  const int nblk = (j1 - j0 + kBlk - 1) / kBlk;
  auto rows_of = [&](int bi) { return [=](int r) { return min(j0 + bi * kBlk + r, j1 - 1); }; };
  // Q is in registers before the ring starts, so that no later wait for it
  // has to cover the ring loads.
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0)
  u32x4 pend = {0u, 0u, 0u, 0u};  // E4M3: the rows of the next block, in registers
  if constexpr (kFp8) {
    store_block_e4m3(ring, load_block_e4m3(kb8, rows_of(0)));
    if (nblk > 1) pend = load_block_e4m3(kb8, rows_of(1));
  } else {
    dma_block_w8(ring, kb, rows_of(0));
    if (nblk > 1) dma_block_w8(ring + kSlotB, kb, rows_of(1));
  }
  // acc[q][r]: row (query i0 + q, head r32), key hk0 + 8(r/4) + 4hh + r%4 of
  // the half starting at hk0.  The running reference m moves only when a
  // logit exceeds it by more than 64 binades: the half's terms are summed
  // against the current m while the next half's MFMAs run (each term at
  // most 2^64, so the sum stays finite and keeps fp32 relative precision);
  // only a sum above 2^64 (or a first half, or one with masked keys) takes
  // the exact path below.
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  auto finish = [&](const f32x16_t (&acc)[2], const float (&lz)[2], int hk0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int P = P0 + q;
      const bool full = hk0 + 32 <= j1 && hk0 + 31 <= P;
      if (full && m[q] != -INFINITY && lz[q] <= 0x1p64f) {
        l[q] += lz[q];
      } else if (full) {
        float bm = acc[q][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) bm = fmaxf(bm, acc[q][r]);
        const float mn = fmaxf(m[q], bm * a.c2);
        float sum = l[q] * fast_exp2(m[q] - mn);
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += fast_exp2(fmaf(acc[q][r], a.c2, -mn));
        l[q] = sum;
        m[q] = mn;
      } else {
        float x[16];
        float bm = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = hk0 + 8 * (r >> 2) + 4 * hh + (r & 3);
          x[r] = (j < j1 && j <= P) ? acc[q][r] * a.c2 : -INFINITY;
          bm = fmaxf(bm, x[r]);
        }
        const float mn = fmaxf(m[q], bm);
        const float mref = (mn == -INFINITY) ? 0.f : mn;
        float sum = l[q] * fast_exp2(m[q] - mref);
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += fast_exp2(x[r] - mref);
        l[q] = sum;
        m[q] = mn;
      }
    }
  };
  f32x16_t prev[2] = {{}, {}};
  int prev_k0 = 0;
  for (int bi = 0; bi < nblk; ++bi) {
    // Block bi has landed for every wave; the slot of block bi-1 is free.
    ring_barrier_w8(bi + 1 < nblk);
    if constexpr (kFp8) {
      // Block bi+1 goes into the slot of block bi-2 (done before the last
      // barrier) and is complete in LDS at the next one.
      if (bi + 1 < nblk) store_block_e4m3(ring + ((bi + 1) % kPfRing) * kSlotB, pend);
      if (bi + 2 < nblk) pend = load_block_e4m3(kb8, rows_of(bi + 2));
    } else {
      if (bi + 2 < nblk) dma_block_w8(ring + ((bi + 2) % kPfRing) * kSlotB, kb, rows_of(bi + 2));
    }
    const uint8_t* kp[8];
    k_opnd_ptrs(ring + (bi % kPfRing) * kSlotB, r32, hh, kp);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16_t cur[2];
      float lz[2] = {0.f, 0.f};
      half_logits<true>(kp, mt, qa, qb, cur, [&](int e) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          lz[0] += fast_exp2(fmaf(prev[0][2 * e + u], a.c2, -m[0]));
          lz[1] += fast_exp2(fmaf(prev[1][2 * e + u], a.c2, -m[1]));
        }
      });
      // The sums are needed here, next to the MFMAs (the compiler would
      // otherwise sink them into the conditional below).
      asm volatile("" ::"v"(lz[0]), "v"(lz[1]));
      if (bi > 0 || mt > 0) finish(prev, lz, prev_k0);
      prev[0] = cur[0];
      prev[1] = cur[1];
      prev_k0 = j0 + bi * kBlk + 32 * mt;
    }
  }
  {
    float lz[2] = {0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      lz[0] += fast_exp2(fmaf(prev[0][r], a.c2, -m[0]));
      lz[1] += fast_exp2(fmaf(prev[1][r], a.c2, -m[1]));
    }
    finish(prev, lz, prev_k0);
  }
  float ma = m[0], la = l[0], mb = m[1], lb = l[1];
  merge_ml(ma, la, __shfl_xor(ma, 32), __shfl_xor(la, 32));
  merge_ml(mb, lb, __shfl_xor(mb, 32), __shfl_xor(lb, 32));
  if (hh == 0) {
    st[r32] = make_float2(ma, la);
    st[32 + r32] = make_float2(mb, lb);
  }
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
template <bool kFp8>
__global__ __launch_bounds__(64 * kPfWaves) void pf_colsum(PfArgs a) {
  const int rb = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  const int N = clamp_ctx(a.ctx_len, b, a.cap);
  const int i0 = rb * 16 + 2 * wave;
  const int P0 = N - a.n_q + i0, P1 = P0 + 1;
  const int P_last = N - a.n_q + rb * 16 + 15;
  const int j0 = s * a.split;
  const int j1 = min(j0 + a.split, P_last + 1);
  if (P_last < 0 || j0 >= j1) {
    // A block entirely before the cache start sees no key: log-sum-exp -inf.
    if (P_last < 0 && s == 0 && a.lse_out != nullptr && hh == 0 && r32 < a.H) {
      a.lse_out[((size_t)b * a.n_q + i0) * a.H + r32] = -INFINITY;
      a.lse_out[((size_t)b * a.n_q + i0 + 1) * a.H + r32] = -INFINITY;
    }
    return;
  }
  // One LDS object: with several, the compiler tracks the ring loads per
  // object and waits for all of them before any read of the ring.  The
  // per-wave column sums rotate over three buffers: a block's second half is
  // summed after the next block's barrier, and its total is formed after the
  // barrier after that.  The totals of the split stay in LDS until the end
  // (no global store inside the loop, whose wait counts only ring loads).
  __shared__ struct __attribute__((aligned(16))) {
    uint8_t ring[kPfRing * kSlotB];
    float s_L[16 * 32];
    float s_cs[3][kPfWaves][kBlk];
    float s_col[kPfSplit];
  } sm;
  uint8_t* ring = sm.ring;
  float* s_L = sm.s_L;
  auto& s_cs = sm.s_cs;
  fold_rows(a, b, rb, N, s_L, s == 0);
  bf16x8_t qa[8], qb[8];
  const uint16_t* qrow = a.q + ((size_t)b * a.n_q + i0) * a.H * kHeadDim;
  load_q(qrow, a.H, r32, hh, P0 >= 0, qa);
  load_q(qrow + a.H * kHeadDim, a.H, r32, hh, P1 >= 0, qb);
  float La[16], Lb[16];  // rows (heads) 8(r/4) + 4hh + r%4 of the two queries
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    La[r] = s_L[(2 * wave) * 32 + 8 * (r >> 2) + 4 * hh + (r & 3)];
    Lb[r] = s_L[(2 * wave + 1) * 32 + 8 * (r >> 2) + 4 * hh + (r & 3)];
  }
  const uint16_t* kb = a.k + (size_t)b * a.kv_stride;
  const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(a.k) + (size_t)b * a.kv_stride;
  float* out = a.colsum + ((size_t)b * (a.n_q / 16) + rb) * a.cap;
  const int nblk = (j1 - j0 + kBlk - 1) / kBlk;
  auto rows_of = [&](int bi) { return [=](int r) { return min(j0 + bi * kBlk + r, j1 - 1); }; };
  // Q is in registers before the ring starts, so that no later wait for it
  // has to cover the ring loads.
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0)
  u32x4 pend = {0u, 0u, 0u, 0u};  // E4M3: the rows of the next block, in registers
  if constexpr (kFp8) {
    store_block_e4m3(ring, load_block_e4m3(kb8, rows_of(0)));
    if (nblk > 1) pend = load_block_e4m3(kb8, rows_of(1));
  } else {
    dma_block_w8(ring, kb, rows_of(0));
    if (nblk > 1) dma_block_w8(ring + kSlotB, kb, rows_of(1));
  }
  auto block_sum = [&](int bj) {
    if (threadIdx.x < kBlk) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kPfWaves; ++w) sum += s_cs[bj % 3][w][threadIdx.x];
      sm.s_col[bj * kBlk + threadIdx.x] = sum;
    }
  };
  // acc[q][r]: row (query i0 + q, head 8(r/4) + 4hh + r%4), key hk0 + r32 of
  // the half starting at hk0.  The column sum over the two queries' 32 head
  // rows: 16 each in this lane, 16 each in lane ^ 32.  Padded heads have
  // L = +inf, so their p is 0.
  auto finish = [&](float ca, float cb, int hb, int hmt) {
    const int j = j0 + hb * kBlk + 32 * hmt + r32;
    if (!(j < j1 && j <= P0)) ca = 0.f;
    if (!(j < j1 && j <= P1)) cb = 0.f;
    float cs = ca + cb;
    cs += __shfl_xor(cs, 32);
    if (hh == 0) s_cs[hb % 3][wave][32 * hmt + r32] = cs;
  };
  f32x16_t prev[2] = {{}, {}};
  for (int bi = 0; bi < nblk; ++bi) {
    ring_barrier_w8(bi + 1 < nblk);
    if constexpr (kFp8) {
      // Block bi+1 goes into the slot of block bi-2 (done before the last
      // barrier) and is complete in LDS at the next one.
      if (bi + 1 < nblk) store_block_e4m3(ring + ((bi + 1) % kPfRing) * kSlotB, pend);
      if (bi + 2 < nblk) pend = load_block_e4m3(kb8, rows_of(bi + 2));
    } else {
      if (bi + 2 < nblk) dma_block_w8(ring + ((bi + 2) % kPfRing) * kSlotB, kb, rows_of(bi + 2));
    }
    if (bi > 1) block_sum(bi - 2);
    const uint8_t* kp[8];
    k_opnd_ptrs(ring + (bi % kPfRing) * kSlotB, r32, hh, kp);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16_t cur[2];
      float ca = 0.f, cb = 0.f;
      half_logits<false>(kp, mt, qa, qb, cur, [&](int e) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          ca += fast_exp2(fmaf(prev[0][2 * e + u], a.c2, -La[2 * e + u]));
          cb += fast_exp2(fmaf(prev[1][2 * e + u], a.c2, -Lb[2 * e + u]));
        }
      });
      asm volatile("" ::"v"(ca), "v"(cb));  // computed next to the MFMAs
      if (mt == 1) finish(ca, cb, bi, 0);
      else if (bi > 0) finish(ca, cb, bi - 1, 1);
      prev[0] = cur[0];
      prev[1] = cur[1];
    }
  }
  {
    float ca = 0.f, cb = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      ca += fast_exp2(fmaf(prev[0][r], a.c2, -La[r]));
      cb += fast_exp2(fmaf(prev[1][r], a.c2, -Lb[r]));
    }
    finish(ca, cb, nblk - 1, 1);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  if (nblk > 1) block_sum(nblk - 2);
  block_sum(nblk - 1);
  __syncthreads();
  for (int t = threadIdx.x; t < j1 - j0; t += 64 * kPfWaves) out[j0 + t] = sm.s_col[t];
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
// P^T: O^T += V^T P^T with p rounded to bf16 (nearest, ties to even), the
// MFMA's operand type: each term's relative error is at most 2^-8, so an
// output moves by at most 2^-8 of sum_j p_j |v_j| beyond the fp32 error.
constexpr int kOutWaves = 8;

template <bool kFp8>
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
    const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(a.k) + (size_t)b * a.kv_stride;
    const uint8_t* vb8 = reinterpret_cast<const uint8_t*>(a.v) + (size_t)b * a.kv_stride;
    const int nblk = (j1 + kBlk - 1) / kBlk;
    auto issue = [&](int bi) {
      auto rows = [=](int r) { return min(bi * kBlk + r, j1 - 1); };
      dma_block_w8(sm.ring[bi % kRing][0], kb, rows);
      dma_block_w8(sm.ring[bi % kRing][1], vb, rows);
    };
    // E4M3: the K and V rows of the next block, in registers.
    u32x4 pk = {0u, 0u, 0u, 0u}, pv = {0u, 0u, 0u, 0u};
    auto load8 = [&](int bi) {
      auto rows = [=](int r) { return min(bi * kBlk + r, j1 - 1); };
      pk = load_block_e4m3(kb8, rows);
      pv = load_block_e4m3(vb8, rows);
    };
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4));  // vmcnt(0) lgkmcnt(0): Q
    if constexpr (kFp8) {
      load8(0);
      store_block_e4m3(sm.ring[0][0], pk);
      store_block_e4m3(sm.ring[0][1], pv);
      if (nblk > 1) load8(1);
    } else {
      issue(0);
      if (nblk > 1) issue(1);
    }
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
      if constexpr (kFp8) {
        // Block bi+1 goes into the slot of block bi-2, done before the last
        // barrier; the barrier after the V transpose publishes it.
        if (bi + 1 < nblk) {
          store_block_e4m3(sm.ring[(bi + 1) % kRing][0], pk);
          store_block_e4m3(sm.ring[(bi + 1) % kRing][1], pv);
        }
        if (bi + 2 < nblk) load8(bi + 2);
      } else {
        if (bi + 2 < nblk) issue(bi + 2);
      }
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
      // Blocks wholly inside the wave's causal range skip the mask.
      auto block = [&](auto masked) {
        constexpr bool kMasked = decltype(masked)::value;
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
            u32x4 pb;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              float pp[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const int r = 8 * sp + 2 * jj + u;
                const int j = kb0 + 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
                const float e = fast_exp2(fmaf(acc[r], a.c2, -Lh));
                pp[u] = (!kMasked || j <= P) ? e : 0.f;
              }
              // v_cvt_pk_bf16_f32: both to bf16, nearest, ties to even.
              pb[jj] = __builtin_bit_cast(
                  uint32_t, __builtin_convertvector((f32x2_t){pp[0], pp[1]}, bf16x2_t));
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const u32x4 av =
                  *reinterpret_cast<const u32x4*>(&sm.vt[32 * t + r32][32 * mt + 16 * sp + 8 * hh]);
              o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(pb), o[t],
                                                             0, 0, 0);
            }
          }
        }
      };
      if (kb0 + kBlk - 1 <= P)
        block(std::false_type{});
      else
        block(std::true_type{});
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
            f32x4{o[t][4 * g] * a.v_scale, o[t][4 * g + 1] * a.v_scale,
                  o[t][4 * g + 2] * a.v_scale, o[t][4 * g + 3] * a.v_scale};
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

template <bool kFp8>
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
  // The list's keys, all read at once (one round trip for both passes).
  __shared__ int s_keys[(kMaxTop + kMaxWindow + kSpWaves + kBlk - 1) / kBlk * kBlk];
  bf16x8_t qr[8];
  load_q(a.q + ((size_t)b * a.n_q + i) * a.H * kHeadDim, a.H, r32, hh, P >= 0, qr);
  for (int p = threadIdx.x; p < total; p += blockDim.x) s_keys[p] = key_of(p);
  __syncthreads();  // every thread's gathers read keys that other threads wrote
  const void* kb = kFp8 ? static_cast<const void*>(reinterpret_cast<const uint8_t*>(a.k) +
                                                   (size_t)b * a.kv_stride)
                        : static_cast<const void*>(a.k + (size_t)b * a.kv_stride);
  const uint16_t* vb = a.v + (size_t)b * a.kv_stride;
  const uint8_t* vb8 = reinterpret_cast<const uint8_t*>(a.v) + (size_t)b * a.kv_stride;

  // K (and in pass B V) rows of list block bi go through registers two blocks
  // ahead: block bi + 2 is loaded while block bi is in the MFMAs, so a
  // block's gather latency overlaps the work of the two before it.
  constexpr int kT = 64 * kSpWaves;
  constexpr int kPieces = kBlk * (kFp8 ? 8 : 16) / kT;  // 16-byte pieces per thread
  static_assert(kPieces >= 1 && kBlk * (kFp8 ? 8 : 16) % kT == 0, "whole pieces");
  const int nblk = (total + kBlk - 1) / kBlk;
  auto key_at = [&](int bi, int r) { return s_keys[min(bi * kBlk + r, total - 1)]; };
  auto load_rows = [&](const void* base, int bi, u32x4 (&x)[kPieces]) {
#pragma unroll
    for (int it = 0; it < kPieces; ++it) {
      const int e = threadIdx.x + it * kT;
      if constexpr (kFp8) {
        const int r = e >> 3, c = e & 7;
        x[it] = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(base) +
                                                (size_t)key_at(bi, r) * kHeadDim + 16 * c);
      } else {
        const int r = e >> 4, c = e & 15;
        x[it] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) +
                                                (size_t)key_at(bi, r) * kHeadDim + 8 * c);
      }
    }
  };
  auto store_k = [&](const u32x4 (&x)[kPieces]) {
#pragma unroll
    for (int it = 0; it < kPieces; ++it) {
      const int e = threadIdx.x + it * kT;
      if constexpr (kFp8) {
        const int r = e >> 3, c = e & 7;
        *reinterpret_cast<u32x4*>(kblk + r * kRowB + 32 * c) = e4m3x8_to_bf16x8(x[it][0], x[it][1]);
        *reinterpret_cast<u32x4*>(kblk + r * kRowB + 32 * c + 16) =
            e4m3x8_to_bf16x8(x[it][2], x[it][3]);
      } else {
        const int r = e >> 4, c = e & 15;
        *reinterpret_cast<u32x4*>(kblk + r * kRowB + 16 * c) = x[it];
      }
    }
  };
  // V block transposed: vt[d][key] (E4M3 rows widened to bf16).
  auto store_v = [&](const u32x4 (&y)[kPieces]) {
#pragma unroll
    for (int it = 0; it < kPieces; ++it) {
      const int e = threadIdx.x + it * kT;
      if constexpr (kFp8) {
        const int r = e >> 3, c = e & 7;
        const u32x4 xs[2] = {e4m3x8_to_bf16x8(y[it][0], y[it][1]),
                             e4m3x8_to_bf16x8(y[it][2], y[it][3])};
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            vt[16 * c + 8 * hf + 2 * u][r] = (uint16_t)(xs[hf][u] & 0xFFFFu);
            vt[16 * c + 8 * hf + 2 * u + 1][r] = (uint16_t)(xs[hf][u] >> 16);
          }
      } else {
        const int r = e >> 4, c = e & 15;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          vt[8 * c + 2 * u][r] = (uint16_t)(y[it][u] & 0xFFFFu);
          vt[8 * c + 2 * u + 1][r] = (uint16_t)(y[it][u] >> 16);
        }
      }
    }
  };

  // Pass A: row statistics over the list.
  float m = -INFINITY, l = 0.f;
  auto pass_a = [&](int bi) {
    const int p0 = bi * kBlk;
    const int* s_key = s_keys + p0;
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
  };
  {
    u32x4 k0[kPieces], k1[kPieces];
    if (nblk > 0) load_rows(kb, 0, k0);
    if (nblk > 1) load_rows(kb, 1, k1);
    for (int bi = 0; bi < nblk; bi += 2) {
      __syncthreads();
      store_k(k0);
      if (bi + 2 < nblk) load_rows(kb, bi + 2, k0);
      __syncthreads();
      pass_a(bi);
      if (bi + 1 >= nblk) break;
      __syncthreads();
      store_k(k1);
      if (bi + 3 < nblk) load_rows(kb, bi + 3, k1);
      __syncthreads();
      pass_a(bi + 1);
    }
  }
  merge_ml(m, l, __shfl_xor(m, 32), __shfl_xor(l, 32));
  const float Lrow = (l > 0.f) ? m + log2f(l) : INFINITY;  // this lane's row (head r32)

  // Pass B: O = sum_j 2^(x - L) v_j.
  f32x16_t o[4] = {{}, {}, {}, {}};
  const void* vsrc = kFp8 ? static_cast<const void*>(vb8) : static_cast<const void*>(vb);
  auto pass_b = [&](int bi) {
    const int p0 = bi * kBlk;
    const int* s_key = s_keys + p0;
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
  };
  {
    u32x4 k0[kPieces], k1[kPieces], v0[kPieces], v1[kPieces];
    if (nblk > 0) {
      load_rows(kb, 0, k0);
      load_rows(vsrc, 0, v0);
    }
    if (nblk > 1) {
      load_rows(kb, 1, k1);
      load_rows(vsrc, 1, v1);
    }
    for (int bi = 0; bi < nblk; bi += 2) {
      __syncthreads();
      store_k(k0);
      store_v(v0);
      if (bi + 2 < nblk) {
        load_rows(kb, bi + 2, k0);
        load_rows(vsrc, bi + 2, v0);
      }
      __syncthreads();
      pass_b(bi);
      if (bi + 1 >= nblk) break;
      __syncthreads();
      store_k(k1);
      store_v(v1);
      if (bi + 3 < nblk) {
        load_rows(kb, bi + 3, k1);
        load_rows(vsrc, bi + 3, v1);
      }
      __syncthreads();
      pass_b(bi + 1);
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
        for (int dt = 0; dt < 4; ++dt)
          orow[(size_t)h * kHeadDim + 32 * dt + r32] = o[dt][r] * a.v_scale;
    }
    if (a.lse_sp != nullptr && hh == 0 && r32 < a.H)
      a.lse_sp[((size_t)b * a.n_q + i) * a.H + r32] = (l > 0.f) ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

}  // namespace

// Logits in base 2 (sm_scale log2(e), times the K cache's scale for E4M3)
// and the factor of the outputs (the V cache's scale for E4M3).
static float logit_scale(const hs2_attn_desc& d) {
  return d.sm_scale * 1.4426950408889634f * (d.dtype == HS2_FP8_E4M3 ? d.k_scale : 1.f);
}
static float value_scale(const hs2_attn_desc& d) {
  return d.dtype == HS2_FP8_E4M3 ? d.v_scale : 1.f;
}

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
  a.c2 = logit_scale(d);
  a.stats = reinterpret_cast<float2*>(ws + w.stats_off);
  a.colsum = reinterpret_cast<float*>(ws + w.colsum_off);
  a.lse_out = lse;
  a.window = d.window;
  const dim3 g(d.n_q / 16, a.nsplit, d.batch);
  if (d.dtype == HS2_FP8_E4M3) {
    pf_stats<true><<<g, 64 * kPfWaves, 0, st>>>(a);
    pf_colsum<true><<<g, 64 * kPfWaves, 0, st>>>(a);
  } else {
    pf_stats<false><<<g, 64 * kPfWaves, 0, st>>>(a);
    pf_colsum<false><<<g, 64 * kPfWaves, 0, st>>>(a);
  }
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
  a.c2 = logit_scale(d);
  a.v_scale = value_scale(d);
  a.stats = reinterpret_cast<float2*>(ws + w.stats_off);
  if (d.dtype == HS2_FP8_E4M3)
    pf_out<true><<<dim3(d.n_q / kOutWaves, d.batch), 512, 0, st>>>(a, o_full);
  else
    pf_out<false><<<dim3(d.n_q / kOutWaves, d.batch), 512, 0, st>>>(a, o_full);
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
  a.c2 = logit_scale(d);
  a.v_scale = value_scale(d);
  a.top_idx = top_idx;
  a.top_cnt = top_cnt;
  a.k_top = d.k_top;
  a.window = d.window;
  a.o = o;
  a.lse_sp = lse;
  if (d.dtype == HS2_FP8_E4M3)
    pf_sparse<true><<<dim3(d.n_q / kSpWaves, d.batch), 64 * kSpWaves, 0, st>>>(a);
  else
    pf_sparse<false><<<dim3(d.n_q / kSpWaves, d.batch), 64 * kSpWaves, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace hs2

