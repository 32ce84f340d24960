// Block-level selection: HySparse's predecessor design, kept beside the
// token-level selector so that the two can be compared at the same budget.
//
// HySparse spends the sparse budget on blocks of 64 consecutive tokens;
// HySparse2 replaces that with single tokens ("HySparse2: How Xiaomi Split
// the Transformer to Fix Agent Prefill Costs", section "KV Reuse and
// Token-Level Sparse Selection"; the paper summary's "KV Reuse refinements"
// compares the two at the same attention budget).  Here a row's pool
// [0, pe) is cut into aligned blocks of `block` tokens (the last one cut at
// pe), a block's importance is the sum of its tokens' fp32 importance,
// rounded once to fp32, and the k_top / block blocks of largest importance
// are taken, ties to the lower block.  Their pool tokens are written in
// ascending order in the token selector's output form, so the sparse layer
// runs on them unchanged.
//
// Piece sums: blk_sums adds each piece of min(block, 32) keys in fp64 with a
// half-wave butterfly, and blk_select adds a 64-key block's two pieces in fp64
// before the one rounding to fp32.  An fp64 sum of at most 64 fp32 values is
// exact whenever their exponents span less than about 23 binades, so then the
// result is the exact sum rounded once, whatever the order of the additions.
// blk_select: one workgroup per row, the row's block importance held in
// registers (a contiguous run of blocks per thread).  The threshold is found
// by an MSB-first radix over d = key - min(key) on the order-preserving
// uint32 image, in digits of at most 12 bits starting at the highest bit
// where the keys differ, so the first digit spreads the keys over the LDS
// histogram instead of piling them into the few bins of one exponent.  Then
// an ordered compaction: exclusive scans give every selected block its rank
// and hand the ties at the threshold to the lowest indices.
#include "select_core.h"

namespace hs2 {
namespace {

constexpr int kBlkSumThreads = 256;

__global__ __launch_bounds__(kBlkSumThreads) void blk_sums(
    const float* __restrict__ scores, int cap, const int32_t* __restrict__ ctx_len, int tiles,
    int n_q, int tile_q, int window, int piece, double* __restrict__ ps, int ps_stride) {
  const int r = blockIdx.y;
  const RowGeom g = row_geom(ctx_len, cap, r, tiles, n_q, tile_q, 0, window);
  const int j0 = blockIdx.x * kBlkSumThreads;
  if (j0 >= g.pe) return;  // uniform over the workgroup
  const int j = j0 + threadIdx.x;
  double x = j < g.pe ? (double)scores[(size_t)r * cap + j] : 0.0;
  for (int off = 1; off < piece; off <<= 1) x += __shfl_xor(x, off);
  if ((j & (piece - 1)) == 0 && j < g.pe) ps[(size_t)r * ps_stride + j / piece] = x;
}

// Block-wide min and max of v (all threads call).
template <int kThreads>
__device__ __forceinline__ void block_min_max(uint32_t& lo, uint32_t& hi, uint32_t* s_lo,
                                              uint32_t* s_hi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, off));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, off));
  }
  if (lane == 0) {
    s_lo[wave] = lo;
    s_hi[wave] = hi;
  }
  __syncthreads();
  lo = s_lo[0];
  hi = s_hi[0];
  for (int w = 1; w < kThreads / 64; ++w) {
    lo = min(lo, s_lo[w]);
    hi = max(hi, s_hi[w]);
  }
  __syncthreads();
}

// One row per workgroup of kThreads; thread t holds blocks
// [kPer t, kPer t + kPer) in registers (kPer * kThreads >= nb).  Block m's
// importance is the fp64 sum of its pieces 2m and 2m + 1 when
// block = 2 * piece, else piece m, rounded to fp32.
template <int kThreads, int kPer>
__global__ __launch_bounds__(kThreads) void blk_select(
    const double* __restrict__ ps, int ps_stride, const int32_t* __restrict__ ctx_len, int cap,
    int tiles, int n_q, int tile_q, int k_top, int window, int block, int piece,
    int32_t* __restrict__ top_idx, int32_t* __restrict__ top_cnt) {
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t scratch[kThreads / 64];
  __shared__ uint32_t scratch2[kThreads / 64];
  __shared__ uint32_t res[2];
  __shared__ int32_t sel[kMaxTop];  // selected blocks, ascending
  const int r = blockIdx.x, t = threadIdx.x;
  const RowGeom g = row_geom(ctx_len, cap, r, tiles, n_q, tile_q, 0, window);
  const int pe = g.pe;
  const int nb = (pe + block - 1) / block;
  const int n_sel = min(k_top / block, nb);
  const double* row = ps + (size_t)r * ps_stride;

  // Order keys of this thread's blocks; 0 marks a slot past the row (every
  // real key is at least 0x80000000, the image of +0).
  uint32_t key[kPer];
  const int m0 = t * kPer;
  if (block == piece) {
#pragma unroll
    for (int i = 0; i < kPer; i += 2) {
      double2 v = make_double2(0.0, 0.0);
      if (m0 + i < nb) v = *reinterpret_cast<const double2*>(row + m0 + i);
      key[i] = (m0 + i < nb) ? order_key((float)v.x) : 0u;
      key[i + 1] = (m0 + i + 1 < nb) ? order_key((float)v.y) : 0u;
    }
  } else {
    // Pieces 2m, 2m + 1; a piece that starts at or past the pool end is 0.
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q0 = 2 * (m0 + i);
      double2 v = make_double2(0.0, 0.0);
      if (m0 + i < nb) v = *reinterpret_cast<const double2*>(row + q0);
      if ((q0 + 1) * piece >= pe) v.y = 0.0;
      key[i] = (m0 + i < nb) ? order_key((float)(v.x + v.y)) : 0u;
    }
  }

  // Keys above `tau` are all taken, and the first `need` keys equal to it.
  // Taking every block: tau below every key; taking none: above every key.
  uint32_t tau = n_sel == 0 ? 0xFFFFFFFFu : 0u, need = 0;
  if (n_sel > 0 && n_sel < nb) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (key[i] != 0u) {
        lo = min(lo, key[i]);
        hi = max(hi, key[i]);
      }
    block_min_max<kThreads>(lo, hi, scratch, scratch2);
    // Radix over d = key - lo from bit `top` down, 12 bits at a time.
    int top = 32 - __clz(hi - lo);  // bits of the largest d (0: all equal)
    uint32_t dpre = 0, mask = 0;
    need = (uint32_t)n_sel;
    while (top > 0) {
      const int sh = max(0, top - 12), nbins = 1 << (top - sh);
      for (int i = t; i < nbins; i += kThreads) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const uint32_t dk = key[i] - lo;
        if (key[i] != 0u && (dk & mask) == dpre)
          atomicAdd(&hist[(dk >> sh) & (uint32_t)(nbins - 1)], 1u);
      }
      __syncthreads();
      find_bin_desc(hist, nbins, need, scratch, res);
      dpre |= res[0] << sh;
      need -= res[1];
      mask |= (uint32_t)(nbins - 1) << sh;
      top = sh;
      __syncthreads();  // every thread has read res before it is rewritten
    }
    tau = lo + dpre;
  }

  // Ordered compaction: ranks from exclusive scans over the threads' runs;
  // the ties at tau go to the lowest blocks.
  uint32_t ties = 0, above = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    ties += key[i] == tau;
    above += key[i] > tau;
  }
  uint32_t total;
  const uint32_t ties_before = block_prefix_sum(ties, scratch, &total);
  uint32_t take = need > ties_before ? min(need - ties_before, ties) : 0u;
  uint32_t rank = block_prefix_sum(above + take, scratch, &total);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    bool in = key[i] > tau;
    if (key[i] == tau && take > 0) {
      in = true;
      --take;
    }
    if (in) sel[rank++] = m0 + i;
  }
  __syncthreads();
  int32_t* out = top_idx + (size_t)r * k_top;
  for (int i = t; i < k_top; i += kThreads) {
    int v = -1;
    if (i < n_sel * block) {
      const int tok = sel[i / block] * block + (i & (block - 1));
      v = tok < pe ? tok : -1;
    }
    out[i] = v;
  }
  if (t == 0) {
    int cnt = n_sel * block;
    if (n_sel > 0 && sel[n_sel - 1] == nb - 1) cnt -= nb * block - pe;
    top_cnt[r] = cnt;
  }
}

}  // namespace

// Row stride of the piece sums (doubles): a multiple of 4, so that rows and
// piece pairs load as 16-byte vectors (the select region's list area holds
// 8 bytes per pool key, at least this).
int blk_stride(int cap, int piece) { return ((cap + piece - 1) / piece + 3) / 4 * 4; }

BlockPieces block_pieces(const hs2_attn_desc& d, int block, int cap, char* sel_ws) {
  const int piece = min(block, 32);
  return BlockPieces{reinterpret_cast<double*>(sel_ws + select_ws(d, cap).list_off), piece,
                     blk_stride(cap, piece)};
}

hipError_t launch_select_blocks(const hs2_attn_desc& d, int block, const float* scores,
                                const int32_t* ctx_len, int cap, int32_t* top_idx,
                                int32_t* top_cnt, char* ws, hipStream_t st) {
  const int tiles = d.n_q / d.tile_q;
  const int rows = d.batch * tiles;
  const BlockPieces pc = block_pieces(d, block, cap, ws);
  blk_sums<<<dim3((cap + kBlkSumThreads - 1) / kBlkSumThreads, rows), kBlkSumThreads, 0, st>>>(
      scores, cap, ctx_len, tiles, d.n_q, d.tile_q, d.window, pc.piece, pc.out, pc.stride);
  const int nb_max = (cap + block - 1) / block;
#define HS2_BLK_SELECT(T, P)                                                                \
  blk_select<T, P><<<rows, T, 0, st>>>(pc.out, pc.stride, ctx_len, cap, tiles, d.n_q, d.tile_q, \
                                       d.k_top, d.window, block, pc.piece, top_idx, top_cnt)
  // 16 waves (a 4-wave workgroup with 16 blocks per thread measured slower
  // on rows of 4,096 blocks: 12.2 against 10.5 us).
  if (nb_max <= 4 * 1024)
    HS2_BLK_SELECT(1024, 4);
  else if (nb_max <= 16 * 1024)
    HS2_BLK_SELECT(1024, 16);
  else
    HS2_BLK_SELECT(1024, 64);
#undef HS2_BLK_SELECT
  return hipGetLastError();
}

}  // namespace hs2
