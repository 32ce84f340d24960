"""Plain fp64 CPU oracle for HySparse2's inner-level KV Reuse hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import or call this module.  It shares no
code with the HIP library (no kernels, headers, helpers or tables) and imports
nothing from it; both sides only read the same seeded input arrays.

Sources (web pages about the preprint "HySparse2: Hybrid Sparse Attention with
Two-Level KV Sharing", arXiv 2609.26368):

* [Summary]  "HySparse2: Hybrid Sparse Attention with Two-Level KV Sharing"
  (academy.dair.ai paper summary): bullets "KV Bridging", "KV Reuse
  refinements", "Inference cost"; Abstract.
* [Origins]  "HySparse2: How Xiaomi Split the Transformer to Fix Agent Prefill
  Costs" (originshq.com): sections "The Self-Decoder and Cross-Decoder Split"
  (with its three projection equations), "KV Reuse and Token-Level Sparse
  Selection", "Limitations and Open Questions".
* [Wire]  "Xiaomi's HySparse2 targets lower computing demands for long-context
  AI agents" (chinaaiwire.com): section "How to interpret the results".

What the pages fix, restated: a full-attention layer attends over the whole
context with one shared K/V head (MQA, [Summary] "Inference cost"; [Wire]
"How to interpret the results") and, besides its own output, yields token
selection indices; the sparse layers that follow reuse those indices and read
the same K/V cache ([Origins] "KV Reuse and Token-Level Sparse Selection").
The selection is 1,024 individual tokens from the whole context plus a forced
window of the 128 most recent tokens (same section; [Summary] "KV Reuse
refinements").  The cross-decoder's K and V are learned projections of a
self-decoder layer's hidden states ([Origins] "The Self-Decoder and
Cross-Decoder Split", first two equations).

Where the pages are silent the oracle takes these readings:

* Importance of key j for a group of queries is the softmax probability of j,
  normalised per (query, head) over that query's whole causal range, summed
  over all query heads and over the group's queries.  A decode step is a group
  of one query; a prefill tile is a group of ``tile_q`` consecutive queries.
* The window tokens are not part of the top-k pool: the pool of a group whose
  first query sits at position P0 is [0, P0 - window + 1), i.e. keys older
  than every window of the group.  The window of a query at P is
  [max(0, P - window + 1), P] (it includes the current token).
* Ties in importance go to the lower key index; the selected indices are
  reported in ascending order.
* Selection is decided on the importance rounded to fp32 (round to nearest
  even); every other quantity stays fp64.
* The softmax scale is an explicit argument (1/sqrt(head_dim) in practice);
  no positional encoding is applied to K.
* HySparse's block-level selection, kept for comparison, ranks aligned
  blocks of the pool by the fp32 sum of their tokens' importance (pairwise
  order), ties to the lower block, at the same token budget and window.
* Query i of a sequence with N cached keys (the new queries' own keys
  included) sits at position N - n_q + i.  A query at a negative position has
  no keys; its output is 0 and its log-sum-exp is -inf.

Parity status: every function here is pinned by tests in
``tests/test_oracle_*.py`` (closed forms, invariants, library routines,
brute force and hand-worked cases); none is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "query_positions",
    "pool_end",
    "attention_probs",
    "full_attn_scores",
    "select_topk_window",
    "block_scores",
    "round_to_f32",
    "select_topk_blocks",
    "selection_set",
    "sparse_attention",
    "dense_attention",
    "swa_attention",
    "bf16_round",
    "fp8_e4m3_value",
    "dequant_kv",
    "bridge_kv",
    "bridge_kv_decode",
]


def _f64(x) -> np.ndarray:
    a = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(a)):
        raise ValueError("oracle inputs must be finite")
    return a


def query_positions(ctx_len: int, n_q: int) -> np.ndarray:
    """Positions of the n_q newest queries in a sequence of ctx_len keys.

    The new queries' own keys are already in the cache (causal
    self-attention sees the current token), so query i sits at
    ctx_len - n_q + i.
    """
    return np.arange(n_q, dtype=np.int64) + (int(ctx_len) - int(n_q))


def pool_end(p0: int, window: int) -> int:
    """End (exclusive) of the top-k pool for a group whose first query is at p0.

    The forced window of the 128 most recent tokens is added on top of the
    1,024 selected ones ([Origins] "KV Reuse and Token-Level Sparse
    Selection"), so window keys are kept out of the pool; for a group, the
    pool holds only keys older than every member's window.
    """
    return max(0, int(p0) - int(window) + 1)


def attention_probs(q_i: np.ndarray, k_vis: np.ndarray, sm_scale: float):
    """Softmax attention probabilities of one query over its visible keys.

    q_i: [H][D] (one query, all heads); k_vis: [n][D] (the single shared KV
    head).  Returns (p [H][n], lse [H]).  This is the full-attention layer's
    attention over the whole (causal) context ([Origins] "KV Reuse and
    Token-Level Sparse Selection").
    """
    q_i = _f64(q_i)
    k_vis = _f64(k_vis)
    n_heads = q_i.shape[0]
    if k_vis.shape[0] == 0:
        return np.zeros((n_heads, 0)), np.full(n_heads, -np.inf)
    s = float(sm_scale) * (q_i @ k_vis.T)          # [H][n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return e / z, (m + np.log(z))[:, 0]


def full_attn_scores(q, k, ctx_len, *, tile_q: int, sm_scale: float, v=None):
    """Full-attention layer of a hybrid block: per-key importance (+ output).

    q: [B][n_q][H][D]; k (and optional v): [B][cap][D]; ctx_len: [B].
    Returns (scores, o_full, lse):

    * scores: float32 [B][n_q // tile_q][cap]; for group t,
      scores[b, t, j] = fp32( sum over queries i of t, heads h, of p_ihj )
      for j < N; entries at j >= N are 0 (the GPU leaves them unwritten).
    * o_full: float64 [B][n_q][H][D], the full layer's own attention output
      sum_j p_ihj v_j (None when v is None).
    * lse: float64 [B][n_q][H], log sum_j exp(s_ihj) over the visible keys.

    The full layer produces both the KV cache and the selection indices
    ([Origins] "KV Reuse and Token-Level Sparse Selection"); the importance
    that drives the selection is the summed probability mass defined in this
    module's header.
    """
    q = _f64(q)
    k = _f64(k)
    vv = None if v is None else _f64(v)
    bsz, n_q, n_heads, head_dim = q.shape
    cap = k.shape[1]
    if n_q % tile_q != 0:
        raise ValueError("n_q must be a multiple of tile_q")
    n_tiles = n_q // tile_q
    scores = np.zeros((bsz, n_tiles, cap), dtype=np.float32)
    o_full = None if vv is None else np.zeros((bsz, n_q, n_heads, head_dim))
    lse = np.full((bsz, n_q, n_heads), -np.inf)
    for b in range(bsz):
        n_keys = int(ctx_len[b])
        if not 0 <= n_keys <= cap:
            raise ValueError("ctx_len out of range")
        pos = query_positions(n_keys, n_q)
        for t in range(n_tiles):
            importance = np.zeros(n_keys)
            for i in range(t * tile_q, (t + 1) * tile_q):
                if pos[i] < 0:
                    continue
                visible = int(pos[i]) + 1
                p, lse[b, i] = attention_probs(q[b, i], k[b, :visible], sm_scale)
                importance[:visible] += p.sum(axis=0)
                if vv is not None:
                    o_full[b, i] = p @ vv[b, :visible]
            scores[b, t, :n_keys] = importance.astype(np.float32)
    return scores, o_full, lse


def select_topk_window(scores, ctx_len, *, n_q: int, tile_q: int, k_top: int,
                       window: int):
    """Selector: the k_top most important pool keys of each query group.

    scores: float32 [B][tiles][cap] (the fp32 importance).  Returns
    (top_idx int32 [B][tiles][k_top], ascending, padded with -1;
    top_cnt int32 [B][tiles]).

    Token-level selection of 1,024 individual keys from the whole context
    ([Origins] "KV Reuse and Token-Level Sparse Selection"; [Summary] "KV Reuse
    refinements").  Order: importance descending, then index ascending; the
    first min(k_top, |pool|) keys are taken and reported in ascending index
    order.  The forced window is not stored here; it is implied by each
    query's position (see ``selection_set``).
    """
    scores = np.asarray(scores, dtype=np.float32)
    bsz, n_tiles, _ = scores.shape
    top_idx = np.full((bsz, n_tiles, k_top), -1, dtype=np.int32)
    top_cnt = np.zeros((bsz, n_tiles), dtype=np.int32)
    for b in range(bsz):
        pos = query_positions(int(ctx_len[b]), n_q)
        for t in range(n_tiles):
            pe = pool_end(pos[t * tile_q], window)
            imp = scores[b, t, :pe]
            if not np.all(np.isfinite(imp)) or np.any(imp < 0):
                raise ValueError("importance must be finite and non-negative")
            idx = np.arange(pe)
            order = np.lexsort((idx, -imp))       # importance desc, index asc
            chosen = np.sort(order[: min(k_top, pe)])
            top_idx[b, t, : chosen.size] = chosen
            top_cnt[b, t] = chosen.size
    return top_idx, top_cnt


def round_to_f32(n: int, e: int) -> np.float32:
    """The float32 nearest to n * 2**e (n >= 0 an integer), ties to even.

    Keeps the top 24 significant bits of n, or fewer where the result falls
    among the float32 subnormals (whose spacing is 2**-149), and rounds the
    dropped bits half to even.
    """
    if n < 0:
        raise ValueError("n must be >= 0")
    if n == 0:
        return np.float32(0.0)
    q = max(e + n.bit_length() - 24, -149)   # exponent of the last kept bit
    if q <= e:
        m = n << (e - q)
    else:
        s = q - e
        m, r = divmod(n, 1 << s)
        half = 1 << (s - 1)
        if r > half or (r == half and m & 1):
            m += 1
        if m == 1 << 24:
            m, q = 1 << 23, q + 1
    if q + 23 > 127:
        raise OverflowError("sum beyond the float32 range")
    return np.float32(math.ldexp(m, q))       # m < 2**24: exact in both formats


def block_scores(imp_pool, block: int) -> np.ndarray:
    """Importance of the aligned blocks of `block` tokens that cover a pool.

    imp_pool: float32 importance of the pool tokens [0, pe).  Block m covers
    tokens [m*block, (m+1)*block) cut at pe; its importance is the sum of its
    tokens' importance.  The pages do not say how HySparse ranks its blocks;
    the summed attention mass is the reading taken, the block analogue of the
    token importance ([Origins] "KV Reuse and Token-Level Sparse Selection":
    HySparse gives the budget to 64-token blocks).  Since the sum decides which
    blocks are taken, it is defined exactly: the exact sum of the tokens'
    float32 values, rounded once to float32 (ties to even).  Every float32 is
    an integer multiple of 2**-149, so the sum is taken over those integers.
    ``block`` is a power of two.
    """
    imp_pool = np.asarray(imp_pool, dtype=np.float32)
    if block < 1 or block & (block - 1):
        raise ValueError("block must be a power of two")
    pe = imp_pool.shape[0]
    nb = -(-pe // block)
    units = imp_pool.astype(np.float64) * 2.0 ** 149   # exact integers in float64
    out = np.empty(nb, dtype=np.float32)
    for m in range(nb):
        n = sum(int(u) for u in units[m * block:min((m + 1) * block, pe)])
        out[m] = round_to_f32(n, -149)
    return out


def select_topk_blocks(scores, ctx_len, *, n_q: int, tile_q: int, k_top: int, window: int,
                       block: int):
    """HySparse's block-level selection, at the same token budget.

    The predecessor design spends the sparse budget on blocks of 64
    consecutive tokens rather than on single tokens ([Origins] "KV Reuse and
    Token-Level Sparse Selection"; [Summary] "KV Reuse refinements", the
    comparison at the same attention budget).  Here: the k_top // block
    blocks of the pool with the largest ``block_scores`` (ties to the lower
    block index) are taken, and their pool tokens are reported in ascending
    order, in the same (top_idx, top_cnt) form as ``select_topk_window``.
    The pool and the forced window are those of the token-level selector, so
    the two differ only in granularity.  A block cut by the pool end holds
    only its pool tokens, so top_cnt can fall below k_top.
    """
    if k_top % block:
        raise ValueError("k_top must be a multiple of block")
    scores = np.asarray(scores, dtype=np.float32)
    bsz, n_tiles, _ = scores.shape
    top_idx = np.full((bsz, n_tiles, k_top), -1, dtype=np.int32)
    top_cnt = np.zeros((bsz, n_tiles), dtype=np.int32)
    for b in range(bsz):
        pos = query_positions(int(ctx_len[b]), n_q)
        for t in range(n_tiles):
            pe = pool_end(pos[t * tile_q], window)
            imp = scores[b, t, :pe]
            if not np.all(np.isfinite(imp)) or np.any(imp < 0):
                raise ValueError("importance must be finite and non-negative")
            bs = block_scores(imp, block)
            order = np.lexsort((np.arange(bs.size), -bs))   # block score desc, index asc
            chosen = np.sort(order[: min(k_top // block, bs.size)])
            toks = [np.arange(m * block, min((m + 1) * block, pe)) for m in chosen]
            toks = np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)
            top_idx[b, t, : toks.size] = toks
            top_cnt[b, t] = toks.size
    return top_idx, top_cnt


def selection_set(top_row, top_cnt: int, p_i: int, window: int) -> np.ndarray:
    """Keys attended by a sparse-layer query at position p_i.

    The selected keys of its group followed by the forced window
    [max(0, p_i - window + 1), p_i] of the most recent tokens, which are
    always present ([Origins] "KV Reuse and Token-Level Sparse Selection").
    The two parts are disjoint and the result is ascending.
    """
    if p_i < 0:
        return np.zeros(0, dtype=np.int64)
    top = np.asarray(top_row[: int(top_cnt)], dtype=np.int64)
    win = np.arange(max(0, int(p_i) - int(window) + 1), int(p_i) + 1)
    return np.concatenate([top, win])


def sparse_attention(q, k, v, ctx_len, top_idx, top_cnt, *, tile_q: int,
                     window: int, sm_scale: float):
    """Sparse layer: attention of each query over its selection set only.

    q: [B][n_q][H][D] (the sparse layer's own query); k, v: [B][cap][D], the
    same cache the full layer used; top_idx/top_cnt from the selector.
    Returns (o float64 [B][n_q][H][D], lse float64 [B][n_q][H]).  The sparse
    layers reuse the full layer's indices and read the same K/V cache, with
    no state of their own ([Origins] "KV Reuse and Token-Level Sparse
    Selection").
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    bsz, n_q, n_heads, head_dim = q.shape
    o = np.zeros((bsz, n_q, n_heads, head_dim))
    lse = np.full((bsz, n_q, n_heads), -np.inf)
    for b in range(bsz):
        pos = query_positions(int(ctx_len[b]), n_q)
        for i in range(n_q):
            t = i // tile_q
            sel = selection_set(top_idx[b, t], top_cnt[b, t], pos[i], window)
            if sel.size == 0:
                continue
            p, lse[b, i] = attention_probs(q[b, i], k[b, sel], sm_scale)
            o[b, i] = p @ v[b, sel]
    return o, lse


def swa_attention(q, k, v, ctx_len, *, window: int, sm_scale: float):
    """Sliding-window attention of the self-decoder's SWA layers.

    The self-decoder, the only part of the model that prefill runs, mixes
    full-attention layers with sliding-window attention layers ([Origins]
    "The Self-Decoder and Cross-Decoder Split"; [Summary] "KV Bridging").
    The pages give no window size for those layers, so it is an argument.  A
    query at position P attends causally to the keys
    [max(0, P - window + 1), P] of its sequence, one shared K/V head:
      o = softmax(sm_scale * q . k) v over that range.
    Returns (o float64 [B][n_q][H][D], lse float64 [B][n_q][H], natural log).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    if window < 1:
        raise ValueError("window must be positive")
    bsz, n_q, n_heads, head_dim = q.shape
    o = np.zeros((bsz, n_q, n_heads, head_dim))
    lse = np.full((bsz, n_q, n_heads), -np.inf)
    for b in range(bsz):
        pos = query_positions(int(ctx_len[b]), n_q)
        for i in range(n_q):
            if pos[i] < 0:
                continue
            lo = max(0, int(pos[i]) - window + 1)
            keys = np.arange(lo, int(pos[i]) + 1)
            p, lse[b, i] = attention_probs(q[b, i], k[b, keys], sm_scale)
            o[b, i] = p @ v[b, keys]
    return o, lse


def dense_attention(q, k, v, ctx_len, *, sm_scale: float):
    """Causal dense attention over the whole context (the full layer's output).

    Same as ``full_attn_scores(..., v=v)[1:]`` but without the importance; it
    is what a sparse layer computes when the budget covers the whole pool.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    bsz, n_q, n_heads, head_dim = q.shape
    o = np.zeros((bsz, n_q, n_heads, head_dim))
    lse = np.full((bsz, n_q, n_heads), -np.inf)
    for b in range(bsz):
        pos = query_positions(int(ctx_len[b]), n_q)
        for i in range(n_q):
            if pos[i] < 0:
                continue
            visible = int(pos[i]) + 1
            p, lse[b, i] = attention_probs(q[b, i], k[b, :visible], sm_scale)
            o[b, i] = p @ v[b, :visible]
    return o, lse


def bf16_round(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and fp32's exponent range.  Rounding is
    done once, directly from the fp64 value (no intermediate fp32 step).
    Returns the rounded values as float64.
    """
    x = np.asarray(x, dtype=np.float64)
    mant, expo = np.frexp(x)                  # x = mant * 2**expo, |mant| in [0.5, 1)
    # Below the smallest normal bfloat16 (2**-126) the spacing is fixed.
    expo = np.maximum(expo, -125)
    scaled = np.ldexp(x, 8 - expo)            # 8 significant bits left of the point
    rounded = np.ldexp(np.round(scaled), expo - 8)   # np.round: ties to even
    big = np.abs(rounded) > 3.3895313892515355e38    # largest finite bfloat16
    return np.where(big, np.copysign(np.inf, x), rounded)


def fp8_e4m3_value(codes) -> np.ndarray:
    """Exact values (float64) of FP8 E4M3 bytes, the KV-cache format the
    pages' cost figures assume ([Origins] "Results": prefill cost with an FP8
    KV cache; [Wire] "How to interpret the results": the FP8 cache sizes).

    The pages do not spell the encoding out; this is the OCP E4M3 layout: a
    sign bit, 4 exponent bits with bias 7 and 3 mantissa bits.  Exponent 0
    holds the subnormals m/8 * 2**-6; S.1111.111 is NaN and there are no
    infinities, so the largest finite value is 1.75 * 2**8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = c >> 7
    expo = (c >> 3) & 15
    mant = c & 7
    mag = np.where(expo == 0, np.ldexp(mant / 8.0, -6), np.ldexp(1.0 + mant / 8.0, expo - 7))
    val = np.where(sign == 1, -mag, mag)
    return np.where((expo == 15) & (mant == 7), np.nan, val)


def dequant_kv(codes, scale) -> np.ndarray:
    """Values of an FP8 K or V cache with one scale per cache: scale * e4m3(x).
    (The pages give no scaling convention; one fp32 scale per cache is the
    reading taken.)"""
    return fp8_e4m3_value(codes) * float(scale)


def bridge_kv(h, w_k, w_v, *, row_chunk: int = 8192):
    """KV Bridging projection: K = H W_K and V = H W_V, rounded to bfloat16.

    h: [M][d_model] hidden states of a self-decoder full-attention layer;
    w_k, w_v: [d_model][head_dim].  The cross-decoder layer's K and V are
    learned projections of those hidden states ([Origins] "The Self-Decoder
    and Cross-Decoder Split", first two equations; [Summary] "KV Bridging").
    Products are summed in fp64 and rounded once to bfloat16 (ties to even).
    Rows are processed in chunks only to bound memory.
    """
    w_k = _f64(w_k)
    w_v = _f64(w_v)
    m_rows = np.asarray(h).shape[0]
    k_out = np.empty((m_rows, w_k.shape[1]))
    v_out = np.empty((m_rows, w_v.shape[1]))
    for r0 in range(0, m_rows, row_chunk):
        hc = _f64(np.asarray(h)[r0:r0 + row_chunk])
        k_out[r0:r0 + row_chunk] = bf16_round(hc @ w_k)
        v_out[r0:r0 + row_chunk] = bf16_round(hc @ w_v)
    return k_out, v_out


def bridge_kv_decode(h, w_k, w_v, pos, k_cache, v_cache):
    """KV Bridging during decode: each sequence's new token gets its
    cross-decoder K and V row from its self-decoder hidden state.

    Prefill skips the cross-decoder, and the cross-decoder's full-attention
    caches are built from self-decoder hidden states ([Origins] "The
    Self-Decoder and Cross-Decoder Split"); a token generated later goes
    through the self-decoder too, so its rows come from the same projection.
    h: [B][d_model]; pos: int [B], the cache row of sequence b's token;
    k_cache, v_cache: [B][cap][head_dim].  Returns copies of the caches with
    row pos[b] of sequence b set to bridge_kv(h[b]); a pos outside [0, cap)
    writes nothing.
    """
    k_new = np.array(k_cache, dtype=np.float64, copy=True)
    v_new = np.array(v_cache, dtype=np.float64, copy=True)
    k_rows, v_rows = bridge_kv(h, w_k, w_v)
    cap = k_new.shape[1]
    for b, p in enumerate(np.asarray(pos)):
        if 0 <= int(p) < cap:
            k_new[b, int(p)] = k_rows[b]
            v_new[b, int(p)] = v_rows[b]
    return k_new, v_new
