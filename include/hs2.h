/*
 * hs2.h -- C ABI of libhs2, the MI355X (gfx950) kernels of HySparse2's
 * inner-level KV Reuse path: token-level sparse attention in which a
 * full-attention MQA layer scores every cached key, a selector keeps the
 * top-k keys plus a forced window of the most recent ones, and the sparse
 * layers that follow attend only to that selection over the same K/V cache.
 * The KV Bridging projection that builds such a cache from self-decoder
 * hidden states is exported too.
 *
 * Sources: web pages about the preprint "HySparse2: Hybrid Sparse Attention
 * with Two-Level KV Sharing" (arXiv 2609.26368):
 *   [Summary] "HySparse2: Hybrid Sparse Attention with Two-Level KV Sharing"
 *             (academy.dair.ai summary), bullets "KV Bridging", "KV Reuse
 *             refinements", "Inference cost".
 *   [Origins] "HySparse2: How Xiaomi Split the Transformer to Fix Agent
 *             Prefill Costs" (originshq.com), sections "The Self-Decoder and
 *             Cross-Decoder Split" (projection equations) and "KV Reuse and
 *             Token-Level Sparse Selection".
 *   [Wire]    "Xiaomi's HySparse2 targets lower computing demands for
 *             long-context AI agents" (chinaaiwire.com), "How to interpret
 *             the results" (MQA).
 * The pages give the operations in prose only; the calls below are this
 * library's own interface to them.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor argument is a DEVICE pointer owned by the caller; the
 *   library never allocates, frees or keeps a pointer after returning, and
 *   never synchronises.  Work is enqueued asynchronously on `stream` (a
 *   hipStream_t; NULL means the default stream).
 * - Arguments are validated on the host before anything is enqueued: a call
 *   that returns HS2_EINVAL, HS2_EUNSUPPORTED, HS2_EALIGN or HS2_EWORKSPACE
 *   has enqueued nothing and written nothing.  HS2_EHIP reports that the HIP
 *   runtime refused a kernel launch; kernels that the same call launched
 *   before it may already be enqueued, so the outputs are then undefined.
 *   Asynchronous device faults surface at the caller's next synchronisation.
 * - Every pointer must be 16-byte aligned (HS2_EALIGN otherwise).
 * - Shapes: B = batch, Q = n_q new queries per sequence, H = query heads,
 *   D = head_dim = 128, one shared K/V head (MQA, [Summary] "Inference
 *   cost"; [Wire] "How to interpret the results").  Layouts are row-major:
 *     q        [B][Q][H][D]      dtype of the descriptor (bf16 for
 *                                HS2_FP8_E4M3)
 *     k, v     [B][cap][D]       dtype of the descriptor; sequence stride
 *                                kv_stride ELEMENTS (>= cap*D), row stride D
 *     ctx_len  int32 [B]         device array: keys held by each sequence,
 *                                the new queries' own keys included;
 *                                values are clamped to [0, cap] on device
 *     scores   f32 [B][Q/tile_q][cap]
 *     top_idx  int32 [B][Q/tile_q][k_top], top_cnt int32 [B][Q/tile_q]
 *     o        f32 [B][Q][H][D],  lse f32 [B][Q][H] (natural log)
 * - Query i of sequence b sits at position P = ctx_len[b] - Q + i; it sees
 *   keys 0..P (causal).  Queries at negative positions output 0 / -inf.
 * - Inputs must be finite.  bf16 values are raw bfloat16 bit patterns; fp8
 *   values are raw OCP FP8 E4M3 bytes (1 sign, 4 exponent bits with bias 7,
 *   3 mantissa bits, subnormals, no infinities; 0x7F/0xFF are NaN).
 * - Calls are reentrant.  A workspace may be shared by calls issued in order
 *   on one stream, never by calls that can run concurrently.
 * - Decode scoring of a bf16 or E4M3 cache (hs2_full_attn_scores without
 *   o_full, and the decode steps) reads K once with one workgroup on each
 *   compute unit, and those workgroups wait for one another.  So two such
 *   calls must not run at the same time on one GPU, whatever their streams
 *   or workspaces.  Waits are bounded (about 1 s), after which the scores of
 *   the sequences concerned are NaN (and the decode steps' selections and
 *   sparse outputs for them are undefined).  Batches larger than the GPU's
 *   compute unit count take a two-pass path with no such wait.
 * - kv_capacity is at most 4,194,304 keys (HS2_EUNSUPPORTED beyond).
 */
#ifndef HS2_H_
#define HS2_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define HS2_API __attribute__((visibility("default")))
#else
#define HS2_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef void* hs2_stream_t; /* a hipStream_t */

typedef enum {
  HS2_OK = 0,
  HS2_EINVAL = 1,       /* null pointer, bad size or inconsistent shape */
  HS2_EUNSUPPORTED = 2, /* valid, but outside what the kernels implement */
  HS2_EALIGN = 3,       /* a pointer is not 16-byte aligned */
  HS2_EWORKSPACE = 4,   /* workspace smaller than hs2_workspace_size() */
  HS2_EHIP = 5          /* the HIP runtime reported an error at enqueue */
} hs2_status;

/*
 * Storage types.  HS2_FP8_E4M3 is the FP8 KV cache that the pages' cost
 * figures assume ([Origins] "Results", prefill cost "(FP8 KV cache)"; [Wire]
 * "How to interpret the results"), whose scaling the pages do not give: here
 * K and V are E4M3 bytes with one fp32 scale per cache (desc->k_scale,
 * desc->v_scale; the value of a byte x is scale * e4m3(x)), q stays bf16
 * and the arithmetic is that of the bf16 path (every E4M3 value is exact in
 * bf16).  Decode and chunked prefill; kv_stride must be a multiple of 16
 * (HS2_EALIGN otherwise).
 */
typedef enum { HS2_F32 = 0, HS2_BF16 = 1, HS2_FP8_E4M3 = 2 } hs2_dtype;

/* Attention problem shared by the scoring, selection and sparse calls. */
typedef struct {
  int batch;      /* B >= 1 */
  int n_q;        /* new queries per sequence: 1 (decode) or a multiple of tile_q;
                     batch * n_q <= 2^24 (HS2_EUNSUPPORTED beyond) */
  int n_heads;    /* query heads, 1..32, all sharing one K/V head (MQA) */
  int head_dim;   /* must be 128 */
  int tile_q;     /* queries per selection group: 1 (decode), or a multiple of 16 for
                     chunked prefill, bf16 or E4M3 K/V (64 in the benchmarks) */
  int k_top;      /* selected keys per group, 0..2048 (1024 in HySparse2) */
  int window;     /* forced recent-token window, 0..2048 (128 in HySparse2) */
  int causal;     /* must be 1 */
  float sm_scale; /* softmax scale, normally 1/sqrt(head_dim) */
  hs2_dtype dtype;/* storage type of q, k and v */
  float k_scale;  /* HS2_FP8_E4M3: scale of the K cache (finite, > 0); else ignored */
  float v_scale;  /* HS2_FP8_E4M3: scale of the V cache (finite, > 0); else ignored */
} hs2_attn_desc;

/* Bytes of device workspace the three attention calls need for this problem
 * and cache capacity (one workspace serves all three when they are issued in
 * order on one stream).  Returns 0 when the descriptor is invalid. */
HS2_API size_t hs2_workspace_size(const hs2_attn_desc* desc, int kv_capacity);

/*
 * Full-attention layer scoring ([Origins] "KV Reuse and Token-Level Sparse
 * Selection": the full layer attends over the whole context and yields the
 * selection indices besides its KV cache).
 *
 * For each query group g (tile_q consecutive queries) of sequence b, writes
 *   scores[b][g][j] = sum over queries i in g, heads h of p_ihj,   j < ctx_len[b]
 * where p_ihj = exp(s_ihj - lse_ih), s_ihj = sm_scale * q_ih . k_j, is query
 * i's softmax probability over its causal range 0..P_i (0 for j > P_i).
 * Entries j >= ctx_len[b] are not written.  Optional outputs: lse, and
 * o_full, the full layer's own attention output, fp32 [B][n_q][n_heads][128]:
 *   o_full[b][i][h][:] = sum_j p_ihj v_j      (times v_scale for E4M3 caches)
 * (zero for a query before the cache start).  o_full needs v (HS2_EINVAL
 * without it).  Decode: the second K pass also streams V, and with bf16 or
 * E4M3 caches the scores are summed over heads in a different order than
 * without o_full (same values up to rounding; fp32 caches: the same bits).
 * Prefill: the scores are the same bits as without o_full, and one more pass
 * over K and V computes the output from the statistics of the first.
 * v may be NULL when o_full is NULL.
 */
HS2_API hs2_status hs2_full_attn_scores(const hs2_attn_desc* desc, const void* q,
                                const void* k, const void* v, int64_t kv_stride,
                                const int32_t* ctx_len, int kv_capacity,
                                float* scores, float* o_full, float* lse,
                                void* ws, size_t ws_bytes, hs2_stream_t stream);

/*
 * Selector ([Origins] "KV Reuse and Token-Level Sparse Selection"; [Summary]
 * "KV Reuse refinements"): for each group g of sequence b, with P0 the
 * position of its first query, the pool is keys [0, max(0, P0 - window + 1))
 * -- the window keys are kept out of it -- and the selection is the
 * min(k_top, pool) pool keys of largest score, ties going to the lower index.
 * Writes them to top_idx[b][g][0..cnt) in ascending index order, pads the
 * rest with -1 and writes cnt to top_cnt[b][g].  The forced window itself is
 * implied by each query's position and is not stored.  Scores must be finite
 * and non-negative (as hs2_full_attn_scores writes them); the result is
 * exactly determined by the fp32 values given.
 */
HS2_API hs2_status hs2_select_topk_window(const hs2_attn_desc* desc, const float* scores,
                                  const int32_t* ctx_len, int kv_capacity,
                                  int32_t* top_idx, int32_t* top_cnt,
                                  void* ws, size_t ws_bytes, hs2_stream_t stream);

/*
 * Block-level selection, the design HySparse2 replaces ([Origins] "KV Reuse
 * and Token-Level Sparse Selection": HySparse gives the sparse budget to
 * blocks of 64 neighbouring tokens; [Summary] "KV Reuse refinements"
 * compares the two at the same attention budget), for comparisons at equal
 * budget.  The pool of each row is that of hs2_select_topk_window; it is cut
 * into aligned blocks of block_size tokens (the last one ends at the pool
 * end).  A block's importance is the fp32 sum of its tokens' scores, added
 * as a balanced pairwise tree over its block_size slots (slot pairs (0,1),
 * (2,3), ... level by level; slots past the pool count 0).  The
 * k_top / block_size blocks of largest importance are taken (ties to the
 * lower block) and their pool tokens written to top_idx in ascending order,
 * -1 padded, with top_cnt their number (below k_top when the cut last block
 * is taken or the pool is small), in the same form as
 * hs2_select_topk_window, so hs2_sparse_attn_gather takes them unchanged.
 * block_size is a power of two, 1..64 (HS2_EINVAL otherwise), dividing k_top
 * (HS2_EINVAL); at most 65,536 blocks per row (HS2_EUNSUPPORTED beyond).
 * Other arguments as for hs2_select_topk_window; same workspace size.
 */
HS2_API hs2_status hs2_select_topk_blocks(const hs2_attn_desc* desc, int block_size,
                                          const float* scores, const int32_t* ctx_len,
                                          int kv_capacity, int32_t* top_idx, int32_t* top_cnt,
                                          void* ws, size_t ws_bytes, hs2_stream_t stream);

/*
 * Sparse layer ([Origins] "KV Reuse and Token-Level Sparse Selection": the
 * sparse layers reuse the full layer's indices and read its K/V cache; the
 * 128 most recent tokens are always part of the selection).  For query i at
 * position P of group g:
 *   S_i = top_idx[b][g][0..top_cnt) ++ [max(0, P - window + 1), P]
 *   o[b][i][h] = sum over j in S_i of softmax_S(sm_scale * q_ih . k_j) v_j
 * and lse[b][i][h] = log sum over S_i of exp(sm_scale * q_ih . k_j) (lse may
 * be NULL).  q is the sparse layer's own query.  top_idx/top_cnt must be as
 * hs2_select_topk_window writes them (ascending, inside the pool).
 */
HS2_API hs2_status hs2_sparse_attn_gather(const hs2_attn_desc* desc, const void* q,
                                  const void* k, const void* v, int64_t kv_stride,
                                  const int32_t* ctx_len, int kv_capacity,
                                  const int32_t* top_idx, const int32_t* top_cnt,
                                  float* o, float* lse, void* ws, size_t ws_bytes,
                                  hs2_stream_t stream);

/*
 * Several sparse layers after one full layer.  Each full-attention layer
 * hands its selection and its K/V cache to the sparse layers that follow it
 * ([Origins] "The Self-Decoder and Cross-Decoder Split", on HySparse's KV
 * Reuse), so n_layers sparse layers attend over the same rows with their own
 * queries.  This call gathers every selected K/V row once for all of them.
 * Decode only (n_q = tile_q = 1), bf16 or E4M3 caches (HS2_EUNSUPPORTED
 * otherwise); 1 <= n_layers <= 64.  q_layers is bf16
 * [n_layers][B][H][D], o_layers fp32 [n_layers][B][H][D], lse_layers
 * (nullable) fp32 [n_layers][B][H].  The results are those of n_layers calls
 * of hs2_sparse_attn_gather, bit for bit.  The workspace (16-byte aligned)
 * needs hs2_sparse_layers_workspace_size bytes.
 */
HS2_API size_t hs2_sparse_layers_workspace_size(const hs2_attn_desc* desc, int n_layers);
HS2_API hs2_status hs2_sparse_attn_gather_layers(const hs2_attn_desc* desc, int n_layers,
                                         const void* q_layers, const void* k, const void* v,
                                         int64_t kv_stride, const int32_t* ctx_len,
                                         int kv_capacity, const int32_t* top_idx,
                                         const int32_t* top_cnt, float* o_layers,
                                         float* lse_layers, void* ws, size_t ws_bytes,
                                         hs2_stream_t stream);

/*
 * One decode step of a hybrid block in a single call: the full layer's
 * scoring (as hs2_full_attn_scores, with q), the selection (as
 * hs2_select_topk_window) and the sparse layer (as hs2_sparse_attn_gather,
 * with q_sparse, or q when q_sparse is NULL).  The outputs are exactly those
 * of the three calls issued in order with the same workspace; on the bf16
 * and E4M3 paths the scoring pass also builds the selector's first histogram, which
 * saves the selector one pass over the scores.  lse_full (the full layer's
 * log-sum-exp) and lse (the sparse layer's) may be NULL.
 */
HS2_API hs2_status hs2_decode_step(const hs2_attn_desc* desc, const void* q,
                                   const void* q_sparse, const void* k, const void* v,
                                   int64_t kv_stride, const int32_t* ctx_len, int kv_capacity,
                                   float* scores, float* lse_full, int32_t* top_idx,
                                   int32_t* top_cnt, float* o, float* lse, void* ws,
                                   size_t ws_bytes, hs2_stream_t stream);

/*
 * The step of hs2_decode_step with the block-level selection of
 * hs2_select_topk_blocks in place of the token-level one: scoring, block
 * selection and the sparse layer, with exactly the outputs of those three
 * calls issued in order with the same workspace.  Arguments as for
 * hs2_decode_step and hs2_select_topk_blocks.
 */
HS2_API hs2_status hs2_decode_step_blocks(const hs2_attn_desc* desc, int block_size,
                                          const void* q, const void* q_sparse, const void* k,
                                          const void* v, int64_t kv_stride,
                                          const int32_t* ctx_len, int kv_capacity, float* scores,
                                          float* lse_full, int32_t* top_idx, int32_t* top_cnt,
                                          float* o, float* lse, void* ws, size_t ws_bytes,
                                          hs2_stream_t stream);

/*
 * hs2_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as hs2_decode_step, without ws and
 * ws_bytes: the step's workspace is a 32 MiB (33,554,432-byte) array that the
 * library holds in the device memory of each GPU it runs on, until the process
 * ends.  The call allocates nothing.  It returns HS2_EWORKSPACE (enqueuing
 * nothing) when hs2_workspace_size(desc, kv_capacity) exceeds 32 MiB.  Every
 * call on one GPU uses that GPU's same array: calls that can overlap on one
 * GPU (other streams, other threads) race and must not be issued.  The first
 * call on a device looks up the array's device address (hipGetSymbolAddress);
 * make that first call outside stream capture.
 */
HS2_API hs2_status hs2_decode_step_noalloc(const hs2_attn_desc* desc, const void* q,
                                           const void* q_sparse, const void* k, const void* v,
                                           int64_t kv_stride, const int32_t* ctx_len,
                                           int kv_capacity, float* scores, float* lse_full,
                                           int32_t* top_idx, int32_t* top_cnt, float* o,
                                           float* lse, hs2_stream_t stream);

/*
 * Sliding-window attention of the self-decoder.  Prefill runs only the
 * self-decoder, which mixes full-attention layers with sliding-window
 * attention layers ([Origins] "The Self-Decoder and Cross-Decoder Split";
 * [Summary] "KV Bridging"); this is the attention of those SWA layers.  Query
 * i of sequence b sits at position P = ctx_len[b] - n_q + i and attends to
 * the keys [max(0, P - window + 1), P] of its sequence:
 *   o[b][i][h] = sum_j softmax(sm_scale * q_bih . k_j) v_j,
 *   lse[b][i][h] = log sum_j exp(sm_scale * q_bih . k_j)   (lse may be NULL);
 * queries at negative positions give 0 and -inf.  desc: batch, n_q >= 1,
 * n_heads 1..32 sharing one K/V head, head_dim 128, window >= 1 (the pages
 * give no SWA window size; 128 in the benchmarks), sm_scale, causal = 1,
 * dtype HS2_BF16 (HS2_EUNSUPPORTED otherwise); tile_q and k_top are not used.
 * Layouts and alignment as for the other calls (q [B][n_q][H][D] bf16, k/v
 * [B][cap][D] bf16 with sequence stride kv_stride).  o is [B][n_q][H][D] in
 * o_dtype: HS2_F32, or HS2_BF16 (rounded to nearest even; the next layer's
 * input format, half the bytes to write); HS2_EINVAL otherwise.  No
 * workspace.
 */
HS2_API hs2_status hs2_swa_attention(const hs2_attn_desc* desc, const void* q, const void* k,
                                     const void* v, int64_t kv_stride, const int32_t* ctx_len,
                                     int kv_capacity, void* o, hs2_dtype o_dtype, float* lse,
                                     hs2_stream_t stream);

/*
 * KV Bridging ([Origins] "The Self-Decoder and Cross-Decoder Split", first two
 * equations; [Summary] "KV Bridging"): the K and V of a cross-decoder
 * full-attention layer are learned projections of a self-decoder
 * full-attention layer's hidden states:
 *   k_out[m][:] = bf16(h[m][:] . w_k),  v_out[m][:] = bf16(h[m][:] . w_v)
 * for m < M, with fp32 accumulation and one round-to-nearest-even.  All
 * bfloat16 on the device: h [M][d_model] with row stride ldh (elements),
 * w_k/w_v [d_model][head_dim] row-major, k_out/v_out [M][head_dim] with row
 * stride ld_kv (elements); columns past head_dim are not written.  head_dim
 * must be 128; d_model a positive multiple of 64; ldh >= d_model and
 * ld_kv >= head_dim, both multiples of 8; pointers 16-byte aligned.
 * Enqueued on `stream`.
 */
HS2_API hs2_status hs2_bridge_kv(const uint16_t* h, int64_t ldh, const uint16_t* w_k,
                         const uint16_t* w_v, uint16_t* k_out, uint16_t* v_out,
                         int64_t ld_kv, int M, int d_model, int head_dim,
                         hs2_stream_t stream);

/*
 * W_K and W_V are static parameters, so they can be packed once into the
 * order in which the projection kernel consumes them; hs2_bridge_kv_packed
 * then streams the packed copy straight into on-chip memory instead of
 * transposing the weights in every workgroup.  Same results as
 * hs2_bridge_kv, bit for bit.
 *
 * Bytes of the packed weights for d_model x head_dim projections (0 if the
 * shape is unsupported).
 */
HS2_API size_t hs2_bridge_packed_bytes(int d_model, int head_dim);

/*
 * Packs w_k and w_v (as for hs2_bridge_kv) into w_packed (device,
 * hs2_bridge_packed_bytes bytes, 16-byte aligned, owned by the caller),
 * enqueued on `stream`.  The packed layout is private to this library.
 */
HS2_API hs2_status hs2_bridge_pack_weights(const uint16_t* w_k, const uint16_t* w_v, int d_model,
                                   int head_dim, uint16_t* w_packed, hs2_stream_t stream);

/* hs2_bridge_kv with weights packed by hs2_bridge_pack_weights for the same d_model. */
HS2_API hs2_status hs2_bridge_kv_packed(const uint16_t* h, int64_t ldh, const uint16_t* w_packed,
                                uint16_t* k_out, uint16_t* v_out, int64_t ld_kv, int M,
                                int d_model, int head_dim, hs2_stream_t stream);

/*
 * KV Bridging during decode.  A token generated after prefill also runs the
 * self-decoder, and the cross-decoder's full-attention caches are projections
 * of the self-decoder's hidden states ([Origins] "The Self-Decoder and
 * Cross-Decoder Split"), so each sequence's new token gets its K and V rows
 * from the same projection as in prefill:
 *   k_cache[r][pos[r]][:] = bf16(h[r][:] . w_k),
 *   v_cache[r][pos[r]][:] = bf16(h[r][:] . w_v)     for r < rows,
 * with fp32 accumulation and one round-to-nearest-even.  h: bf16 [rows][d_model]
 * (row stride ldh elements), row r being sequence r's new token; w_packed:
 * weights packed by hs2_bridge_pack_weights for this d_model; pos: device
 * int32 [rows], the cache row of each sequence's token (a value outside
 * [0, kv_capacity) writes nothing for that sequence); k_cache, v_cache: bf16
 * [rows][kv_capacity][head_dim] with sequence stride kv_stride elements.  Only
 * those rows are written.  head_dim 128, d_model a positive multiple of 64
 * (HS2_EUNSUPPORTED otherwise); ldh >= d_model and kv_stride >=
 * kv_capacity * 128, both multiples of 8; pointers 16-byte aligned.
 */
HS2_API hs2_status hs2_bridge_kv_decode(const uint16_t* h, int64_t ldh, const uint16_t* w_packed,
                                        int rows, int d_model, int head_dim, const int32_t* pos,
                                        uint16_t* k_cache, uint16_t* v_cache, int64_t kv_stride,
                                        int kv_capacity, hs2_stream_t stream);

/* Static description of a status code. */
HS2_API const char* hs2_status_string(hs2_status status);

#ifdef __cplusplus
}
#endif

#endif /* HS2_H_ */
