// Block-level selection: HySparse's predecessor design, kept beside the
// token-level selector so that the two can be compared at the same budget.
//
// HySparse spends the sparse budget on blocks of 64 consecutive tokens;
// HySparse2 replaces that with single tokens ("HySparse2: How Xiaomi Split
// the Transformer to Fix Agent Prefill Costs", section "KV Reuse and
// Token-Level Sparse Selection"; the paper summary's "KV Reuse refinements"
// compares the two at the same attention budget).  Here a row's pool
// [0, pe) is cut into aligned blocks of `block` tokens (the last one cut at
// pe), a block's importance is the fp32 sum of its tokens' importance in a
// balanced pairwise order (slot pairs (0,1), (2,3), ... level by level; slots
// past the pool hold 0), and the k_top / block blocks of largest importance
// are taken, ties to the lower block.  Their pool tokens are written in
// ascending order in the token selector's output form, so the sparse layer
// runs on them unchanged.
//
// blk_sums: one thread per token slot, the pairwise tree as an xor butterfly
// inside the wave (x + partner is the same value on both lanes of a pair, so
// the butterfly is exactly the pairwise tree).
// blk_select: one workgroup per row; the threshold block importance by an
// MSB-first radix over the order-preserving uint32 image (four 8-bit
// digits), then an ordered compaction (each thread owns a contiguous run of
// blocks; exclusive scans give every selected block its rank and hand the
// ties at the threshold to the lowest indices).
#include "select_core.h"

namespace hs2 {
namespace {

constexpr int kBlkSumThreads = 256;
constexpr int kBlkSelThreads = 1024;

__global__ __launch_bounds__(kBlkSumThreads) void blk_sums(
    const float* __restrict__ scores, int cap, const int32_t* __restrict__ ctx_len, int tiles,
    int n_q, int tile_q, int window, int block, float* __restrict__ bs, int nb_stride) {
  const int r = blockIdx.y;
  const RowGeom g = row_geom(ctx_len, cap, r, tiles, n_q, tile_q, 0, window);
  const int j0 = blockIdx.x * kBlkSumThreads;
  if (j0 >= g.pe) return;  // uniform over the workgroup
  const int j = j0 + threadIdx.x;
  float x = j < g.pe ? scores[(size_t)r * cap + j] : 0.f;
  for (int off = 1; off < block; off <<= 1) x += __shfl_xor(x, off);
  if ((j & (block - 1)) == 0 && j < g.pe) bs[(size_t)r * nb_stride + j / block] = x;
}

__global__ __launch_bounds__(kBlkSelThreads) void blk_select(
    const float* __restrict__ bs, int nb_stride, const int32_t* __restrict__ ctx_len, int cap,
    int tiles, int n_q, int tile_q, int k_top, int window, int block,
    int32_t* __restrict__ top_idx, int32_t* __restrict__ top_cnt) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scratch[kBlkSelThreads / 64];
  __shared__ uint32_t res[2];
  __shared__ int32_t sel[kMaxTop];  // selected blocks, ascending
  const int r = blockIdx.x, t = threadIdx.x;
  const RowGeom g = row_geom(ctx_len, cap, r, tiles, n_q, tile_q, 0, window);
  const int pe = g.pe;
  const int nb = (pe + block - 1) / block;
  const int n_sel = min(k_top / block, nb);
  const float* row = bs + (size_t)r * nb_stride;

  // Keys above `tau` are all taken, and the first `need` keys equal to it.
  // Taking every block: tau below every key; taking none: above every key.
  uint32_t tau = n_sel == 0 ? 0xFFFFFFFFu : 0u, need = 0;
  if (n_sel > 0 && n_sel < nb) {
    uint32_t mask = 0;
    need = (uint32_t)n_sel;
    for (int d = 3; d >= 0; --d) {
      const int sh = 8 * d;
      for (int i = t; i < 256; i += kBlkSelThreads) hist[i] = 0u;
      __syncthreads();
      for (int m = t; m < nb; m += kBlkSelThreads) {
        const uint32_t key = order_key(row[m]);
        if ((key & mask) == tau) atomicAdd(&hist[(key >> sh) & 255u], 1u);
      }
      __syncthreads();
      find_bin_desc(hist, 256, need, scratch, res);
      tau |= res[0] << sh;
      need -= res[1];
      mask |= 255u << sh;
      __syncthreads();  // every thread has read res before it is rewritten
    }
  }

  // Ordered compaction over contiguous runs of blocks.
  const int per = (nb + kBlkSelThreads - 1) / kBlkSelThreads;
  const int m0 = min(nb, t * per), m1 = min(nb, m0 + per);
  uint32_t ties = 0;
  for (int m = m0; m < m1; ++m) ties += order_key(row[m]) == tau;
  uint32_t total;
  const uint32_t ties_before = block_prefix_sum(ties, scratch, &total);
  uint32_t take = need > ties_before ? need - ties_before : 0u;
  take = min(take, ties);
  uint32_t mine = 0;
  for (int m = m0; m < m1; ++m) {
    const uint32_t key = order_key(row[m]);
    mine += key > tau;
  }
  mine += take;
  uint32_t rank = block_prefix_sum(mine, scratch, &total);
  for (int m = m0; m < m1; ++m) {
    const uint32_t key = order_key(row[m]);
    bool in = key > tau;
    if (key == tau && take > 0) {
      in = true;
      --take;
    }
    if (in) sel[rank++] = m;
  }
  __syncthreads();
  int32_t* out = top_idx + (size_t)r * k_top;
  for (int i = t; i < k_top; i += kBlkSelThreads) {
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

int blk_stride(int cap, int block) { return (cap + block - 1) / block; }

hipError_t launch_select_blocks(const hs2_attn_desc& d, int block, const float* scores,
                                const int32_t* ctx_len, int cap, int32_t* top_idx,
                                int32_t* top_cnt, char* ws, hipStream_t st) {
  const SelectWs w = select_ws(d, cap);
  const int tiles = d.n_q / d.tile_q;
  const int rows = d.batch * tiles;
  const int nbs = blk_stride(cap, block);
  float* bs = reinterpret_cast<float*>(ws + w.list_off);  // rows x nbs floats
  blk_sums<<<dim3((cap + kBlkSumThreads - 1) / kBlkSumThreads, rows), kBlkSumThreads, 0, st>>>(
      scores, cap, ctx_len, tiles, d.n_q, d.tile_q, d.window, block, bs, nbs);
  blk_select<<<rows, kBlkSelThreads, 0, st>>>(bs, nbs, ctx_len, cap, tiles, d.n_q, d.tile_q,
                                              d.k_top, d.window, block, top_idx, top_cnt);
  return hipGetLastError();
}

}  // namespace hs2
