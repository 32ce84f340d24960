"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against a closed form, an invariant, a library
routine, a brute-force evaluation or a hand-worked case, so that a plausible
mistake (a dropped term, a wrong sign or index, a transposed operand, an
off-by-one window or pool) fails at least one of them.
"""

import json
import math
from fractions import Fraction
import os

import numpy as np
import pytest
import scipy.special

import oracle
from workloads import WORKLOADS, make_decode_inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def _closed_form(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"e": math.e}))


def _hand_cases():
    with open(os.path.join(HERE, "golden", "hand_cases.json")) as f:
        return json.load(f)["cases"]


def _hand_inputs(case):
    keys = np.asarray(case["keys"], dtype=np.float64)
    n = keys.size
    q = np.asarray(case["q"], dtype=np.float64)[None, :, :, None]   # [1][n_q][H][1]
    k = keys[None, :, None]
    v = (10.0 * np.arange(1, n + 1))[None, :, None]
    return q, k, v, np.array([n])


@pytest.mark.parametrize("case", _hand_cases(), ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    q, k, v, ctx = _hand_inputs(case)
    n_q, tile_q = case["n_q"], case["tile_q"]
    kt, win = case["k_top"], case["window"]
    scores, _, _ = oracle.full_attn_scores(q, k, ctx, tile_q=tile_q, sm_scale=1.0)
    if "importance" in case:
        want = np.array([_closed_form(x) for x in case["importance"]])
        np.testing.assert_allclose(scores[0, 0], want, rtol=1e-6)
    p0 = oracle.query_positions(ctx[0], n_q)[0]
    assert oracle.pool_end(p0, win) == case["pool_end"]
    top_idx, top_cnt = oracle.select_topk_window(
        scores, ctx, n_q=n_q, tile_q=tile_q, k_top=kt, window=win)
    for t, want_top in enumerate(case["top"]):
        assert top_cnt[0, t] == len(want_top)
        assert list(top_idx[0, t, : top_cnt[0, t]]) == want_top
        assert np.all(top_idx[0, t, top_cnt[0, t]:] == -1)
    pos = oracle.query_positions(ctx[0], n_q)
    for i, want_sel in enumerate(case["selection"]):
        t = i // tile_q
        sel = oracle.selection_set(top_idx[0, t], top_cnt[0, t], pos[i], win)
        assert list(sel) == want_sel
    o, _ = oracle.sparse_attention(q, k, v, ctx, top_idx, top_cnt,
                                   tile_q=tile_q, window=win, sm_scale=1.0)
    for i, expr in enumerate(case.get("o", [])):
        assert o[0, i, 0, 0] == pytest.approx(_closed_form(expr), rel=1e-12)
    if "o_dense" in case:
        od, _ = oracle.dense_attention(q, k, v, ctx, sm_scale=1.0)
        assert od[0, 0, 0, 0] == pytest.approx(_closed_form(case["o_dense"][0]), rel=1e-12)


@pytest.mark.parametrize("case", [c for c in _hand_cases() if "o_dense" in c],
                         ids=lambda c: c["name"])
def test_full_layer_output_hand_cases(case):
    # The full layer's own output (full_attn_scores with v) against the
    # hand-worked dense output of the same case.
    q, k, v, ctx = _hand_inputs(case)
    _, o_full, lse = oracle.full_attn_scores(q, k, ctx, tile_q=case["tile_q"], sm_scale=1.0, v=v)
    assert o_full[0, 0, 0, 0] == pytest.approx(_closed_form(case["o_dense"][0]), rel=1e-12)


def test_full_layer_output_invariants():
    # One visible key: the output is its V row.  Constant V: the output is
    # that constant (the probabilities sum to one).  Two keys with logits
    # a and b: the output is the logistic mix of their V rows.
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 2, 1, 3, 8), _rand(rng, 2, 40, 8), _rand(rng, 2, 40, 8)
    ctx = np.array([1, 40])
    _, o, _ = oracle.full_attn_scores(q, k, ctx, tile_q=1, sm_scale=0.3, v=v)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0], (3, 8)), rtol=0, atol=0)
    _, oc, _ = oracle.full_attn_scores(q, k, ctx, tile_q=1, sm_scale=0.3,
                                       v=np.full_like(v, 2.5))
    np.testing.assert_allclose(oc[1, 0], 2.5, rtol=1e-14)
    ctx2 = np.array([2, 2])
    _, o2, _ = oracle.full_attn_scores(q, k, ctx2, tile_q=1, sm_scale=0.3, v=v)
    for b in range(2):
        for h in range(3):
            a = 0.3 * float(q[b, 0, h] @ k[b, 0])
            c = 0.3 * float(q[b, 0, h] @ k[b, 1])
            w0 = scipy.special.expit(a - c)
            np.testing.assert_allclose(o2[b, 0, h], w0 * v[b, 0] + (1 - w0) * v[b, 1],
                                       rtol=1e-12)


def test_full_layer_output_causal_per_query():
    # Prefill: query i of a block sits at P_i = N - n_q + i and its output is
    # the softmax-weighted V over keys 0..P_i only (scipy's softmax over the
    # scaled logits); a query before the cache start sees no key: output 0
    # and log-sum-exp -inf.
    rng = np.random.default_rng(12)
    n_q, heads, d = 4, 2, 8
    for n in (6, 2):
        q, k, v = _rand(rng, 1, n_q, heads, d), _rand(rng, 1, n, d), _rand(rng, 1, n, d)
        _, o, lse = oracle.full_attn_scores(q, k, np.array([n]), tile_q=n_q, sm_scale=0.5, v=v)
        for i in range(n_q):
            p_i = n - n_q + i
            for h in range(heads):
                if p_i < 0:
                    assert np.all(o[0, i, h] == 0.0) and lse[0, i, h] == -np.inf
                    continue
                s = 0.5 * (k[0, :p_i + 1] @ q[0, i, h])
                want = scipy.special.softmax(s) @ v[0, :p_i + 1]
                np.testing.assert_allclose(o[0, i, h], want, rtol=1e-12, atol=1e-14)
                assert lse[0, i, h] == pytest.approx(scipy.special.logsumexp(s), rel=1e-13)


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def test_importance_sums_to_heads_decode():
    # Each head's probabilities sum to one, so the summed importance is H.
    rng = np.random.default_rng(1)
    q, k = _rand(rng, 3, 1, 5, 16), _rand(rng, 3, 300, 16)
    ctx = np.array([300, 17, 1])
    s, _, _ = oracle.full_attn_scores(q, k, ctx, tile_q=1, sm_scale=0.25)
    for b in range(3):
        assert s[b, 0, : ctx[b]].astype(np.float64).sum() == pytest.approx(5.0, rel=1e-6)
        assert np.all(s[b, 0, ctx[b]:] == 0)
        assert np.all(s[b, 0, : ctx[b]] >= 0) and np.all(s[b, 0] <= 5.0)


def test_importance_sums_to_tile_heads_prefill():
    rng = np.random.default_rng(2)
    n_q, tile_q, heads = 8, 4, 3
    q, k = _rand(rng, 1, n_q, heads, 8), _rand(rng, 1, 40, 8)
    s, _, _ = oracle.full_attn_scores(q, k, np.array([40]), tile_q=tile_q, sm_scale=0.5)
    for t in range(n_q // tile_q):
        assert s[0, t].astype(np.float64).sum() == pytest.approx(tile_q * heads, rel=1e-6)
        # causal: the tile's last query sits at 40 - 8 + 4t + 3; nothing later is seen
        last = 40 - n_q + t * tile_q + tile_q - 1
        assert np.all(s[0, t, last + 1:] == 0)


def test_identical_keys_give_uniform_importance():
    # Closed form: equal logits give p = 1/N per head, so I = H/N exactly.
    rng = np.random.default_rng(3)
    k = np.tile(rng.standard_normal(128), (4096, 1))[None]
    q = rng.standard_normal((1, 1, 32, 128))
    s, _, _ = oracle.full_attn_scores(q, k, np.array([4096]), tile_q=1, sm_scale=1 / math.sqrt(128))
    assert np.all(s[0, 0] == np.float32(32 / 4096))
    top, cnt = oracle.select_topk_window(s, [4096], n_q=1, tile_q=1, k_top=1024, window=128)
    assert cnt[0, 0] == 1024 and np.array_equal(top[0, 0], np.arange(1024))


def test_single_head_is_textbook_softmax():
    # Library routine: scipy's softmax of the scaled logits.
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((1, 1, 1, 32)), rng.standard_normal((1, 700, 32))
    s, _, lse = oracle.full_attn_scores(q, k, np.array([700]), tile_q=1, sm_scale=0.3)
    logits = 0.3 * (k[0] @ q[0, 0, 0])
    np.testing.assert_allclose(s[0, 0], scipy.special.softmax(logits), rtol=2e-7)
    assert lse[0, 0, 0] == pytest.approx(scipy.special.logsumexp(logits), rel=1e-13)


def _brute_force(q, k, v, ctx, n_q, tile_q, k_top, window, scale):
    """Element-by-element evaluation with Python floats and math.exp."""
    bsz, _, heads, dim = q.shape
    out_scores, out_top, out_o = {}, {}, {}
    for b in range(bsz):
        n = int(ctx[b])
        pos = [n - n_q + i for i in range(n_q)]
        for t in range(n_q // tile_q):
            imp = [0.0] * n
            for i in range(t * tile_q, (t + 1) * tile_q):
                if pos[i] < 0:
                    continue
                for h in range(heads):
                    lg = [scale * sum(float(q[b, i, h, d]) * float(k[b, j, d]) for d in range(dim))
                          for j in range(pos[i] + 1)]
                    mx = max(lg)
                    z = sum(math.exp(x - mx) for x in lg)
                    for j in range(pos[i] + 1):
                        imp[j] += math.exp(lg[j] - mx) / z
            imp32 = [float(np.float32(x)) for x in imp]
            out_scores[b, t] = imp32
            pe = max(0, pos[t * tile_q] - window + 1)
            ranked = sorted(range(pe), key=lambda j: (-imp32[j], j))
            out_top[b, t] = sorted(ranked[:k_top])
            for i in range(t * tile_q, (t + 1) * tile_q):
                if pos[i] < 0:
                    out_o[b, i] = [[0.0] * dim for _ in range(heads)]
                    continue
                sel = out_top[b, t] + list(range(max(0, pos[i] - window + 1), pos[i] + 1))
                rows = []
                for h in range(heads):
                    lg = [scale * sum(float(q[b, i, h, d]) * float(k[b, j, d]) for d in range(dim))
                          for j in sel]
                    mx = max(lg)
                    w = [math.exp(x - mx) for x in lg]
                    z = sum(w)
                    rows.append([sum(w[a] * float(v[b, j, d]) for a, j in enumerate(sel)) / z
                                 for d in range(dim)])
                out_o[b, i] = rows
    return out_scores, out_top, out_o


@pytest.mark.parametrize("n_q,tile_q", [(1, 1), (4, 2), (6, 3)])
def test_brute_force_tiny(n_q, tile_q):
    rng = np.random.default_rng(5 + n_q)
    bsz, heads, dim, cap = 2, 3, 4, 23
    q = rng.standard_normal((bsz, n_q, heads, dim))
    k = rng.standard_normal((bsz, cap, dim))
    v = rng.standard_normal((bsz, cap, dim))
    ctx = np.array([23, 11])
    k_top, window, scale = 5, 3, 0.7
    s, _, _ = oracle.full_attn_scores(q, k, ctx, tile_q=tile_q, sm_scale=scale)
    top, cnt = oracle.select_topk_window(s, ctx, n_q=n_q, tile_q=tile_q, k_top=k_top, window=window)
    o, _ = oracle.sparse_attention(q, k, v, ctx, top, cnt, tile_q=tile_q, window=window, sm_scale=scale)
    bs, bt, bo = _brute_force(q, k, v, ctx, n_q, tile_q, k_top, window, scale)
    for (b, t), imp in bs.items():
        np.testing.assert_array_equal(s[b, t, : ctx[b]], np.asarray(imp, dtype=np.float32))
        assert list(top[b, t, : cnt[b, t]]) == bt[b, t]
    for (b, i), rows in bo.items():
        np.testing.assert_allclose(o[b, i], np.asarray(rows), rtol=1e-12, atol=1e-13)


def test_selection_equals_stable_argsort_and_invariants():
    # Library routine: a stable argsort of -I gives the (I desc, index asc) order.
    rng = np.random.default_rng(6)
    w = WORKLOADS["decode_bf16_64k_b16"].replace(batch=3)
    inp = make_decode_inputs(w, ctx_lens=[5000, 1200, 1100], capacity=5000)
    s, _, _ = oracle.full_attn_scores(inp["q"], inp["k"], inp["ctx_len"], tile_q=1,
                                      sm_scale=w.sm_scale)
    # Quantise some scores so that many exact ties exist.
    s = (np.round(s * 2e4) / 2e4).astype(np.float32)
    top, cnt = oracle.select_topk_window(s, inp["ctx_len"], n_q=1, tile_q=1,
                                         k_top=1024, window=128)
    for b, n in enumerate(inp["ctx_len"]):
        pe = n - 128
        order = np.argsort(-s[b, 0, :pe], kind="stable")
        want = np.sort(order[: min(1024, pe)])
        got = top[b, 0, : cnt[b, 0]]
        assert np.array_equal(got, want)
        sel = oracle.selection_set(top[b, 0], cnt[b, 0], n - 1, 128)
        assert sel.size == min(n, 1152)                       # |S| = min(N, K + W)
        assert np.all(np.diff(sel) > 0)                       # ascending, disjoint
        assert set(range(n - 128, n)) <= set(sel.tolist())    # window always present
        assert got.size == 0 or got.max() < pe                # T inside the pool
    del rng


@pytest.mark.parametrize("name", ["decode_f32_4k", "decode_bf16_64k_b16"])
def test_planted_needles_are_selected(name):
    w = WORKLOADS[name]
    n = 4096 if name == "decode_f32_4k" else 8192
    w = w.replace(batch=2, ctx_len=n)
    inp = make_decode_inputs(w)
    s, _, _ = oracle.full_attn_scores(inp["q"], inp["k"], inp["ctx_len"], tile_q=1,
                                      sm_scale=w.sm_scale)
    top, cnt = oracle.select_topk_window(s, inp["ctx_len"], n_q=1, tile_q=1,
                                         k_top=w.k_top, window=w.window)
    for b in range(2):
        assert set(inp["planted"][b].tolist()) <= set(top[b, 0, : cnt[b, 0]].tolist())


def test_clustered_keys_are_selected():
    w = WORKLOADS["decode_bf16_256k_b4"].replace(batch=1, ctx_len=65536)
    inp = make_decode_inputs(w)
    assert inp["planted"][0].size == 262
    s, _, _ = oracle.full_attn_scores(inp["q"], inp["k"], inp["ctx_len"], tile_q=1,
                                      sm_scale=w.sm_scale)
    top, cnt = oracle.select_topk_window(s, inp["ctx_len"], n_q=1, tile_q=1,
                                         k_top=1024, window=128)
    assert set(inp["planted"][0].tolist()) <= set(top[0, 0, : cnt[0, 0]].tolist())


def test_budget_covering_pool_gives_dense_attention():
    # k_top >= |pool| means every key is attended: the textbook softmax.
    rng = np.random.default_rng(7)
    q, k, v = rng.standard_normal((2, 1, 4, 8)), rng.standard_normal((2, 50, 8)), rng.standard_normal((2, 50, 8))
    ctx = np.array([50, 30])
    s, _, _ = oracle.full_attn_scores(q, k, ctx, tile_q=1, sm_scale=0.4)
    top, cnt = oracle.select_topk_window(s, ctx, n_q=1, tile_q=1, k_top=64, window=5)
    o, lse = oracle.sparse_attention(q, k, v, ctx, top, cnt, tile_q=1, window=5, sm_scale=0.4)
    for b in range(2):
        n = ctx[b]
        lg = 0.4 * np.einsum("hd,jd->hj", q[b, 0], k[b, :n])
        want = scipy.special.softmax(lg, axis=1) @ v[b, :n]
        np.testing.assert_allclose(o[b, 0], want, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[b, 0], scipy.special.logsumexp(lg, axis=1), rtol=1e-13)
    od, _ = oracle.dense_attention(q, k, v, ctx, sm_scale=0.4)
    np.testing.assert_allclose(o, od, rtol=1e-12, atol=1e-14)


def test_single_selected_key_returns_its_value():
    # |S| = 1: the output is exactly that key's value row.
    rng = np.random.default_rng(8)
    q, k, v = rng.standard_normal((1, 1, 3, 8)), rng.standard_normal((1, 10, 8)), rng.standard_normal((1, 10, 8))
    ctx = np.array([10])
    s, _, _ = oracle.full_attn_scores(q, k, ctx, tile_q=1, sm_scale=1.0)
    top, cnt = oracle.select_topk_window(s, ctx, n_q=1, tile_q=1, k_top=1, window=0)
    assert cnt[0, 0] == 1
    j = int(top[0, 0, 0])
    assert j == int(np.lexsort((np.arange(10), -s[0, 0]))[0])
    o, _ = oracle.sparse_attention(q, k, v, ctx, top, cnt, tile_q=1, window=0, sm_scale=1.0)
    for h in range(3):
        assert np.array_equal(o[0, 0, h], v[0, j])
    o1, _ = oracle.sparse_attention(q, k, v, np.array([1]), np.full((1, 1, 1), -1), np.zeros((1, 1), int),
                                    tile_q=1, window=4, sm_scale=1.0)
    assert np.array_equal(o1[0, 0, 0], v[0, 0])


def test_equal_logits_average_selected_values():
    rng = np.random.default_rng(9)
    k = np.zeros((1, 40, 8))
    q, v = rng.standard_normal((1, 1, 2, 8)), rng.standard_normal((1, 40, 8))
    ctx = np.array([40])
    s, _, _ = oracle.full_attn_scores(q, k, ctx, tile_q=1, sm_scale=1.0)
    top, cnt = oracle.select_topk_window(s, ctx, n_q=1, tile_q=1, k_top=6, window=4)
    o, _ = oracle.sparse_attention(q, k, v, ctx, top, cnt, tile_q=1, window=4, sm_scale=1.0)
    sel = list(range(6)) + list(range(36, 40))
    np.testing.assert_allclose(o[0, 0, 0], v[0, sel].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_one_query_tiles_reduce_to_decode():
    # A prefill group of one query is a decode step at that query's position.
    rng = np.random.default_rng(10)
    n_q, heads, dim, n = 5, 3, 8, 60
    q, k, v = rng.standard_normal((1, n_q, heads, dim)), rng.standard_normal((1, n, dim)), rng.standard_normal((1, n, dim))
    s, of, lse = oracle.full_attn_scores(q, k, np.array([n]), tile_q=1, sm_scale=0.5, v=v)
    top, cnt = oracle.select_topk_window(s, [n], n_q=n_q, tile_q=1, k_top=7, window=4)
    o, _ = oracle.sparse_attention(q, k, v, [n], top, cnt, tile_q=1, window=4, sm_scale=0.5)
    for i in range(n_q):
        ni = n - n_q + i + 1
        sd, ofd, lsed = oracle.full_attn_scores(q[:, i:i + 1], k, np.array([ni]), tile_q=1, sm_scale=0.5, v=v)
        np.testing.assert_array_equal(sd[0, 0, :ni], s[0, i, :ni])
        np.testing.assert_allclose(ofd[0, 0], of[0, i], rtol=1e-13)
        td, cd = oracle.select_topk_window(sd, [ni], n_q=1, tile_q=1, k_top=7, window=4)
        assert np.array_equal(td[0, 0], top[0, i])
        od, _ = oracle.sparse_attention(q[:, i:i + 1], k, v, [ni], td, cd, tile_q=1, window=4, sm_scale=0.5)
        np.testing.assert_allclose(od[0, 0], o[0, i], rtol=1e-13)


def test_prefill_group_pool_and_selection_sizes():
    # |S_i| = min(K, pool) + min(W, P_i + 1) for every query of a group.
    rng = np.random.default_rng(11)
    n_q, tile_q, n = 16, 8, 300
    q, k = rng.standard_normal((1, n_q, 2, 8)), rng.standard_normal((1, n, 8))
    s, _, _ = oracle.full_attn_scores(q, k, np.array([n]), tile_q=tile_q, sm_scale=0.5)
    top, cnt = oracle.select_topk_window(s, [n], n_q=n_q, tile_q=tile_q, k_top=100, window=32)
    pos = oracle.query_positions(n, n_q)
    for i in range(n_q):
        t = i // tile_q
        pe = pos[t * tile_q] - 32 + 1
        sel = oracle.selection_set(top[0, t], cnt[0, t], pos[i], 32)
        assert sel.size == min(100, pe) + min(32, pos[i] + 1)
        assert np.all(np.diff(sel) > 0) and top[0, t, : cnt[0, t]].max() < pe


def test_queries_before_the_cache_start_are_empty():
    q = np.ones((1, 4, 1, 2))
    k = np.ones((1, 8, 2))
    v = np.arange(16.0).reshape(1, 8, 2)
    s, _, lse = oracle.full_attn_scores(q, k, np.array([2]), tile_q=2, sm_scale=1.0)
    # ctx 2, n_q 4: positions -2, -1, 0, 1; group 0 is empty, group 1 sees keys 0..1
    assert np.all(s[0, 0] == 0) and np.isneginf(lse[0, :2]).all()
    assert s[0, 1, :2].sum() == pytest.approx(2.0)
    top, cnt = oracle.select_topk_window(s, [2], n_q=4, tile_q=2, k_top=3, window=1)
    o, _ = oracle.sparse_attention(q, k, v, [2], top, cnt, tile_q=2, window=1, sm_scale=1.0)
    assert np.all(o[0, :2] == 0)
    assert np.array_equal(o[0, 2, 0], v[0, 0]) and np.array_equal(o[0, 3, 0], v[0, 1])


def test_bf16_round_matches_torch_on_fp32_values():
    # Library routine: torch's fp32 -> bfloat16 conversion rounds to nearest even.
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 100000),
                        np.float32([0.0, -0.0, 1e-40, -3e-39, 3.3e38, -3.4e38])]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_round(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_bf16_round_ties_and_single_rounding():
    u = 2.0 ** -8                                   # half an ulp of bfloat16 at 1.0
    assert oracle.bf16_round(1 + u) == 1.0                      # tie -> even
    assert oracle.bf16_round(1 + 3 * u) == 1 + 4 * u            # tie -> even (up)
    assert oracle.bf16_round(1 + u + 2.0 ** -30) == 1 + 2 * u   # above the tie: up,
    # which a detour through fp32 would miss (fp32 drops the 2**-30 first).
    assert oracle.bf16_round(-(1 + u + 2.0 ** -30)) == -(1 + 2 * u)
    assert np.isinf(oracle.bf16_round(3.4e38))


def test_generator_bf16_bits_match_torch():
    torch = pytest.importorskip("torch")
    from workloads import bf16_bits, bf16_bits_to_f32
    rng = np.random.default_rng(13)
    x = (rng.standard_normal(50000) * 100).astype(np.float32)
    bits = bf16_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, want)
    np.testing.assert_array_equal(bf16_bits_to_f32(bits),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_bridge_is_exact_integer_product():
    # Small integers: every product and sum is exact and representable in
    # bfloat16, so K and V must equal the integer matrix product.
    rng = np.random.default_rng(14)
    h = rng.integers(-3, 4, size=(37, 24))
    wk = rng.integers(-2, 3, size=(24, 5))
    wv = rng.integers(-2, 3, size=(24, 5))
    k, v = oracle.bridge_kv(h.astype(float), wk.astype(float), wv.astype(float), row_chunk=8)
    want_k = [[sum(int(h[r, c]) * int(wk[c, d]) for c in range(24)) for d in range(5)] for r in range(37)]
    want_v = [[sum(int(h[r, c]) * int(wv[c, d]) for c in range(24)) for d in range(5)] for r in range(37)]
    assert np.array_equal(k, np.asarray(want_k, dtype=float))
    assert np.array_equal(v, np.asarray(want_v, dtype=float))


def test_bridge_rounds_the_fp64_product_once():
    rng = np.random.default_rng(15)
    h = rng.standard_normal((100, 64))
    wk, wv = rng.standard_normal((64, 16)), rng.standard_normal((64, 16))
    k, v = oracle.bridge_kv(h, wk, wv, row_chunk=33)
    exact_k = h @ wk
    # within half a bfloat16 ulp of the exact product, and on the bfloat16 grid
    ulp = 2.0 ** (np.floor(np.log2(np.abs(exact_k))) - 7)
    assert np.all(np.abs(k - exact_k) <= ulp / 2)
    assert np.array_equal(oracle.bf16_round(k), k)
    assert v.shape == (100, 16)


# --- FP8 E4M3 KV cache (the format of the pages' cost figures) ----------------

def test_e4m3_known_codes():
    # Code points of the OCP E4M3 encoding: zero, the subnormal range, the
    # smallest normal, 1, 1.5, 2, the largest finite value, NaN.
    v = oracle.fp8_e4m3_value(np.arange(256, dtype=np.uint8))
    assert v[0x00] == 0.0 and np.signbit(v[0x80]) and v[0x80] == 0.0
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6
    assert v[0x38] == 1.0 and v[0x3C] == 1.5 and v[0x40] == 2.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.sum(np.isnan(v)) == 2


def test_e4m3_is_ordered_and_symmetric():
    v = oracle.fp8_e4m3_value(np.arange(256, dtype=np.uint8))
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                 # codes 0x00..0x7E ascend
    assert np.array_equal(v[0x80:0xFF], -pos)       # sign bit mirrors
    # Steps between neighbouring codes: 2**-9 through the subnormals and the
    # first binade, then doubling every 8 codes (3 mantissa bits).
    for c in range(0x7E):
        e = max(c >> 3, 1)
        assert pos[c + 1] - pos[c] == 2.0 ** (e - 10), hex(c)


def test_e4m3_matches_torch_float8():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.fp8_e4m3_value(codes)
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), ~fin)
    assert np.array_equal(got[fin], ref[fin])


def test_dequant_kv_fixed_values():
    # Printed values of the E4M3 format (bias 7): 0x38 = 1.0, 0x3C = 1.5,
    # 0x30 = 0.5, 0x08 = 2^-6 (smallest normal), 0x01 = 2^-9 (smallest
    # subnormal), 0x7E = 448 (largest finite); the sign bit mirrors each.  A byte
    # x of a cache with scale s stands for s * e4m3(x) (the one-scale-per-cache
    # reading), computed in float64 from the float32 scale.
    s = np.float32(0.0103)
    table = {0x38: 1.0, 0x3C: 1.5, 0x30: 0.5, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
             0x7E: 448.0, 0x00: 0.0}
    codes = np.array([list(table) + [c | 0x80 for c in table]], dtype=np.uint8)
    want = [v * float(s) for v in table.values()] + [-v * float(s) for v in table.values()]
    got = oracle.dequant_kv(codes, s)
    assert got.dtype == np.float64
    assert got[0].tolist() == want
    assert np.signbit(got[0, len(table) - 1 + len(table)])      # 0x80 is -0
    # Scaling is linear in the scale and exact for powers of two.
    assert oracle.dequant_kv(np.array([[0x7E]], np.uint8), 0.25)[0, 0] == 112.0
    assert oracle.dequant_kv(np.array([[0x01]], np.uint8), 2.0 ** 9)[0, 0] == 1.0


# --- Block-level selection (HySparse's 64-token blocks, for comparison) -----

def test_block_scores_are_exact_sums_rounded_once():
    # A block's importance is the exact sum of its tokens' float32 scores,
    # rounded once to float32, ties to even.  Sums that float32 holds exactly
    # come out exact, and a block cut by the pool end counts only its tokens.
    x = np.array([1, 2, 3, 4, 5, 6, 7, 8, 9, 10], dtype=np.float32)
    assert oracle.block_scores(x, 4).tolist() == [10.0, 26.0, 19.0]
    assert oracle.block_scores(x, 1).tolist() == x.tolist()
    assert oracle.block_scores(x, 16).tolist() == [55.0]
    t = np.float32(2.0 ** -24)
    # [1, t, t, 0] is exactly 1 + 2^-23, a float32.  Float32 additions left to
    # right, or in the pairwise tree (1 + t) + (t + 0), give 1 instead, since
    # 1 + t is a tie that rounds to 1.
    y = np.array([1.0, t, t, 0.0], dtype=np.float32)
    assert oracle.block_scores(y, 4)[0] == np.float32(1.0 + 2.0 ** -23)
    seq = np.float32(0.0)
    for v in y:
        seq = np.float32(seq + v)
    tree = np.float32(np.float32(y[0] + y[1]) + np.float32(y[2] + y[3]))
    assert seq == tree == np.float32(1.0)
    # 1 + 3t lies halfway between 1 + 2^-23 (odd significand) and 1 + 2^-22:
    # the even one.  1 + t lies halfway between 1 and 1 + 2^-23: 1.
    assert oracle.block_scores(np.array([1.0, t, t, t], np.float32), 4)[0] == \
        np.float32(1.0 + 2.0 ** -22)
    assert oracle.block_scores(np.array([1.0, t], np.float32), 2)[0] == np.float32(1.0)
    # Subnormals add exactly.
    d = np.float32(2.0 ** -149)
    assert oracle.block_scores(np.array([d, d, d], np.float32), 4)[0] == np.float32(3 * 2.0 ** -149)
    # Random scores: where math.fsum is exact (its float64 equals the exact
    # rational sum), numpy's float64 -> float32 cast is the single rounding.
    rng = np.random.default_rng(40)
    z = (rng.random(64 * 50) * 10.0 ** rng.integers(-6, 1, 64 * 50)).astype(np.float32)
    got = oracle.block_scores(z, 64)
    checked = 0
    for m in range(50):
        blk = z[m * 64:(m + 1) * 64]
        f = math.fsum(float(v) for v in blk)
        if Fraction(f) == sum(Fraction(float(v)) for v in blk):
            assert got[m] == np.float32(f)
            checked += 1
    assert checked >= 40
    with pytest.raises(ValueError):
        oracle.block_scores(x, 3)


def test_round_to_f32_matches_the_library_cast():
    # n * 2^e with n < 2^53 is a float64 exactly; numpy's cast to float32 rounds
    # it once, to nearest even, including into the subnormal range.
    rng = np.random.default_rng(43)
    for _ in range(3000):
        n = int(rng.integers(0, 2 ** 53))
        e = int(rng.integers(-210, 40))
        assert oracle.round_to_f32(n, e) == np.float32(math.ldexp(float(n), e)), (n, e)
    for n, e in ((2 ** 24 + 1, -24), (2 ** 24 + 3, -24), (3, -150), (1, -150), (5, -151)):
        assert oracle.round_to_f32(n, e) == np.float32(math.ldexp(float(n), e)), (n, e)
    assert oracle.round_to_f32(0, 0) == np.float32(0.0)


def test_block_selection_hand_case():
    # Decode, ctx 12, window 2: pool [0, 10); blocks of 4: {0..3}, {4..7},
    # {8, 9} (cut by the pool end).  Scores per block: 10, 26, 19.
    s = np.zeros((1, 1, 12), dtype=np.float32)
    s[0, 0, :10] = np.arange(1, 11)
    ctx = np.array([12])
    top, cnt = oracle.select_topk_blocks(s, ctx, n_q=1, tile_q=1, k_top=4, window=2, block=4)
    assert cnt.tolist() == [[4]] and top[0, 0].tolist() == [4, 5, 6, 7]
    top, cnt = oracle.select_topk_blocks(s, ctx, n_q=1, tile_q=1, k_top=8, window=2, block=4)
    assert cnt.tolist() == [[6]]
    assert top[0, 0].tolist() == [4, 5, 6, 7, 8, 9, -1, -1]
    # Equal block scores go to the lower block.
    s[0, 0, :10] = [1, 1, 1, 1, 2, 1, 1, 0, 2, 2]       # blocks 4, 4, 4
    top, cnt = oracle.select_topk_blocks(s, ctx, n_q=1, tile_q=1, k_top=8, window=2, block=4)
    assert top[0, 0].tolist() == [0, 1, 2, 3, 4, 5, 6, 7]
    # Budget beyond the pool: every pool token once.
    top, cnt = oracle.select_topk_blocks(s, ctx, n_q=1, tile_q=1, k_top=16, window=2, block=4)
    assert cnt.tolist() == [[10]] and top[0, 0, :10].tolist() == list(range(10))
    with pytest.raises(ValueError):
        oracle.select_topk_blocks(s, ctx, n_q=1, tile_q=1, k_top=6, window=2, block=4)


def test_block_size_one_is_token_selection():
    rng = np.random.default_rng(41)
    s = rng.integers(0, 6, size=(3, 2, 700)).astype(np.float32) / 8   # many ties
    ctx = np.array([700, 450, 129])
    for kw in (dict(n_q=1, tile_q=1), dict(n_q=64, tile_q=32)):
        n_tiles = kw["n_q"] // kw["tile_q"]
        a = oracle.select_topk_blocks(s[:, :n_tiles], ctx, k_top=64, window=128, block=1, **kw)
        b = oracle.select_topk_window(s[:, :n_tiles], ctx, k_top=64, window=128, **kw)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_block_selection_brute_force_and_invariants():
    # Exactly one set of n blocks has every member ahead of every non-member
    # under (score desc, index asc); it must be the one selected.
    import itertools

    rng = np.random.default_rng(42)
    for trial in range(40):
        block = int(rng.choice([2, 4, 8]))
        n_sel = int(rng.integers(1, 4))
        ctx = int(rng.integers(3, 40))
        window = int(rng.integers(0, 5))
        s = (rng.integers(0, 4, size=(1, 1, ctx)) / 4).astype(np.float32)
        top, cnt = oracle.select_topk_blocks(s, np.array([ctx]), n_q=1, tile_q=1,
                                             k_top=n_sel * block, window=window, block=block)
        pe = max(0, ctx - window)
        nb = -(-pe // block)
        score = [sum(float(v) for v in s[0, 0, m * block:min((m + 1) * block, pe)])
                 for m in range(nb)]   # small dyadic values: every sum is exact
        ahead = lambda a, b: score[a] > score[b] or (score[a] == score[b] and a < b)  # noqa: E731
        sets = [c for c in itertools.combinations(range(nb), min(n_sel, nb))
                if all(ahead(a, b) for a in c for b in range(nb) if b not in c)]
        assert len(sets) == 1
        want = [j for m in sets[0] for j in range(m * block, min((m + 1) * block, pe))]
        c = int(cnt[0, 0])
        assert top[0, 0, :c].tolist() == want, trial
        assert np.all(top[0, 0, c:] == -1)


def test_identical_scores_select_the_first_blocks():
    s = np.full((1, 1, 5000), 0.25, dtype=np.float32)
    top, cnt = oracle.select_topk_blocks(s, np.array([5000]), n_q=1, tile_q=1, k_top=1024,
                                         window=128, block=64)
    assert cnt.tolist() == [[1024]] and top[0, 0].tolist() == list(range(1024))


# --- Sliding-window attention of the self-decoder ----------------------------

def test_swa_hand_case():
    # D = 1, one head, keys 1..5 (scale 1), values 10..50, window 2: the query
    # at position 4 sees keys 3 and 4 (values 4 and 5 for k, 40 and 50 for v).
    k = np.arange(1.0, 6.0)[None, :, None]
    v = (10.0 * np.arange(1, 6))[None, :, None]
    q = np.array([[[[1.0]], [[0.5]]]])                   # queries at positions 3, 4
    o, lse = oracle.swa_attention(q, k, v, np.array([5]), window=2, sm_scale=1.0)
    # position 3: keys 3, 4 (k = 3, 4) with q = 1; position 4: keys 4, 5 with q = 0.5
    w3 = np.array([math.exp(3.0), math.exp(4.0)])
    w4 = np.array([math.exp(2.0), math.exp(2.5)])
    assert o[0, 0, 0, 0] == pytest.approx((w3 @ [30.0, 40.0]) / w3.sum(), rel=1e-14)
    assert o[0, 1, 0, 0] == pytest.approx((w4 @ [40.0, 50.0]) / w4.sum(), rel=1e-14)
    assert lse[0, 0, 0] == pytest.approx(math.log(w3.sum()), rel=1e-14)
    assert lse[0, 1, 0] == pytest.approx(math.log(w4.sum()), rel=1e-14)


def test_swa_wide_window_is_scipy_causal_softmax():
    rng = np.random.default_rng(60)
    q = rng.standard_normal((2, 5, 3, 8))
    k = rng.standard_normal((2, 40, 8))
    v = rng.standard_normal((2, 40, 8))
    ctx = np.array([40, 23])
    o, lse = oracle.swa_attention(q, k, v, ctx, window=10_000, sm_scale=0.3)
    for b in range(2):
        for i in range(5):
            P = ctx[b] - 5 + i
            for h in range(3):
                s = 0.3 * k[b, : P + 1] @ q[b, i, h]
                assert np.allclose(o[b, i, h], scipy.special.softmax(s) @ v[b, : P + 1],
                                   rtol=1e-12, atol=1e-12)
                assert lse[b, i, h] == pytest.approx(scipy.special.logsumexp(s), rel=1e-12)


def test_swa_window_one_returns_own_value_and_brute_force():
    rng = np.random.default_rng(61)
    q = rng.standard_normal((1, 6, 2, 4))
    k = rng.standard_normal((1, 30, 4))
    v = rng.standard_normal((1, 30, 4))
    ctx = np.array([30])
    o, lse = oracle.swa_attention(q, k, v, ctx, window=1, sm_scale=0.5)
    for i in range(6):
        P = 24 + i
        assert np.array_equal(o[0, i], np.repeat(v[0, P][None], 2, axis=0))
        assert np.allclose(lse[0, i], 0.5 * q[0, i] @ k[0, P], rtol=1e-14)
    # brute force with math.exp, window 7
    o, lse = oracle.swa_attention(q, k, v, ctx, window=7, sm_scale=0.5)
    for i in range(6):
        P = 24 + i
        for h in range(2):
            ws = [math.exp(0.5 * sum(q[0, i, h, d] * k[0, j, d] for d in range(4)))
                  for j in range(P - 6, P + 1)]
            tot = sum(ws)
            for d in range(4):
                want = sum(w * v[0, j, d] for w, j in zip(ws, range(P - 6, P + 1))) / tot
                assert o[0, i, h, d] == pytest.approx(want, rel=1e-12, abs=1e-12)
            assert lse[0, i, h] == pytest.approx(math.log(tot), rel=1e-12)


def test_swa_queries_before_the_cache_start_are_empty():
    q = np.ones((1, 4, 1, 2))
    k = np.ones((1, 8, 2))
    v = np.ones((1, 8, 2))
    o, lse = oracle.swa_attention(q, k, v, np.array([2]), window=3, sm_scale=1.0)
    assert np.all(o[0, :2] == 0) and np.all(np.isneginf(lse[0, :2]))
    assert np.all(o[0, 2:] == 1) and np.all(np.isfinite(lse[0, 2:]))


def test_bridge_decode_writes_only_the_token_rows():
    # Small integers: every product and sum is exact, so the rows are the
    # integer products (all representable in bf16 here).
    h = np.array([[1.0, 2.0, 0.0, -1.0], [0.0, 1.0, 1.0, 1.0], [3.0, 0.0, 0.0, 0.0]])
    w_k = np.arange(8.0).reshape(4, 2)
    w_v = -np.arange(8.0).reshape(4, 2)
    k_cache = np.full((3, 5, 2), 9.0)
    v_cache = np.full((3, 5, 2), -9.0)
    k_new, v_new = oracle.bridge_kv_decode(h, w_k, w_v, np.array([4, 0, 5]), k_cache, v_cache)
    assert k_new[0, 4].tolist() == [1 * 0 + 2 * 2 + 0 * 4 - 1 * 6, 1 * 1 + 2 * 3 + 0 * 5 - 1 * 7]
    assert v_new[0, 4].tolist() == [2.0, 0.0]
    assert k_new[1, 0].tolist() == [2 + 4 + 6, 3 + 5 + 7]
    # sequence 2's position is past the cache: nothing written
    assert np.array_equal(k_new[2], k_cache[2]) and np.array_equal(v_new[2], v_cache[2])
    untouched = np.ones((3, 5), bool)
    untouched[0, 4] = untouched[1, 0] = False
    assert np.all(k_new[untouched] == 9.0) and np.all(v_new[untouched] == -9.0)
    # the rows equal the bulk projection
    k_rows, v_rows = oracle.bridge_kv(h, w_k, w_v)
    assert np.array_equal(k_new[0, 4], k_rows[0]) and np.array_equal(v_new[1, 0], v_rows[1])
