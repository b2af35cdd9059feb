"""Pins of the fp64 oracle against facts fixed outside it: hand-worked
examples, closed forms, textbook special cases (dense / sink+window softmax
attention via torch's SDPA), a per-token brute force, invariants of the
subtraction form, the first-order-Taylor order of the linear part, and the
recurrence."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _params(**kw):
    base = dict(num_q_heads=1, num_kv_heads=1, head_dim=4, block_size=4, top_k=2,
                num_sink=1, window=4, linear_tail=1, scale=0.0)
    base.update(kw)
    return O.Params(**base)


def _poly_e(c):
    return sum(ci * math.e ** i for i, ci in enumerate(c))


# ----------------------------------------------------------------------------
# Hand-worked examples
# ----------------------------------------------------------------------------

def test_golden_block_score():
    ex = json.load(open(GOLDEN))["block_score"]
    K = np.array(ex["keys"], float)
    mean, var = O.block_statistics(K, ex["block_size"])
    np.testing.assert_array_equal(mean[0], ex["mean"])
    np.testing.assert_array_equal(var[0], ex["var"])
    sc = O.block_score(np.array(ex["q"], float), mean, var, ex["scale"])
    t = ex["score_terms"]
    assert sc[0] == pytest.approx(t["const"] + math.log(t["log_num"] / t["log_den"]), rel=1e-15)


def test_golden_selection_and_exact_set():
    ex = json.load(open(GOLDEN))["selection"]
    p = _params(block_size=ex["block_size"], num_sink=ex["num_sink"], window=ex["window"])
    cands = O.candidate_blocks(ex["T"], p)
    assert cands.tolist() == ex["candidates"]
    for case in ex["cases"]:
        sel = O.select_top_k(cands, np.array(case["scores"]), case["k"])
        assert sel.tolist() == case["selected"], case
    E = O.exact_token_mask(ex["T"], ex["exact_set"]["selected"], p)
    assert np.flatnonzero(E).tolist() == ex["exact_set"]["E"]
    assert np.flatnonzero(~E).tolist() == ex["exact_set"]["U"]


def test_golden_straddling_block():
    ex = json.load(open(GOLDEN))["straddle"]
    p = _params(block_size=ex["block_size"], num_sink=ex["num_sink"], window=ex["window"])
    assert O.candidate_blocks(ex["T"], p).tolist() == ex["candidates"]
    E = O.exact_token_mask(ex["T"], ex["selected"], p)
    assert np.flatnonzero(E).tolist() == ex["E"]
    assert np.flatnonzero(~E).tolist() == ex["U"]


@pytest.mark.parametrize("form", ["definition", "subtraction"])
@pytest.mark.parametrize("linear", [1, 0])
def test_golden_decode(form, linear):
    ex = json.load(open(GOLDEN))["decode"]
    p = O.Params(num_q_heads=1, num_kv_heads=1, head_dim=1, block_size=ex["block_size"],
                 top_k=ex["top_k"], num_sink=ex["num_sink"], window=ex["window"],
                 linear_tail=linear, scale=ex["scale"])
    K = np.array(ex["keys"], float)[:, None]
    V = np.array(ex["values"], float)[:, None]
    st = O.global_state(K, V)
    assert st.S[0, 0] == ex["state"]["S"] and st.z[0] == ex["state"]["z"]
    assert st.sv[0] == ex["state"]["sv"] and st.n == ex["state"]["n"]
    r = O.decode_head(np.array(ex["q"]), K, V, p, form=form)
    assert r.selected.tolist() == ex["selected"]
    np.testing.assert_allclose(r.scores, ex["scores"], rtol=0, atol=1e-15)
    key = "out_linear_on" if linear else "out_linear_off"
    want = _poly_e(ex[key]["num_poly_in_e"]) / _poly_e(ex[key]["den_poly_in_e"])
    assert r.out[0] == pytest.approx(want, rel=1e-14)
    if linear:
        assert r.num_u[0] == pytest.approx(ex["num_u"], abs=1e-12)
        assert r.den_u == pytest.approx(ex["den_u"], abs=1e-12)


# ----------------------------------------------------------------------------
# Stored formats and grouping
# ----------------------------------------------------------------------------

def test_bf16_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x8000], np.uint16)
    want = [1.0, -2.0, 1.0078125, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, -0.0]
    assert O.to_f64(bits, "bf16").tolist() == want


def test_generator_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -3.0], np.float32)
    assert W.bf16_round(x).tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC040]


def test_gqa_grouping_is_contiguous():
    p = _params(num_q_heads=8, num_kv_heads=2)
    assert [O.kv_head_of(h, p) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]


# ----------------------------------------------------------------------------
# Statistics and score
# ----------------------------------------------------------------------------

def test_block_stats_arithmetic_progression():
    B, d = 16, 3
    a = np.array([0.5, -2.0, 7.0])
    delta = np.array([0.25, 3.0, -1.0])
    blk = a[None, :] + np.arange(B)[:, None] * delta[None, :]
    K = np.concatenate([blk, blk + 10.0, np.ones((B, d)) * 4.0, np.ones((5, d))])  # 3 full blocks + ragged tail
    mean, var = O.block_statistics(K, B)
    assert mean.shape == (3, d)
    np.testing.assert_allclose(mean[0], a + delta * (B - 1) / 2, rtol=1e-15)
    np.testing.assert_allclose(mean[1], a + 10 + delta * (B - 1) / 2, rtol=1e-15)
    np.testing.assert_allclose(var[0], delta ** 2 * (B * B - 1) / 12, rtol=1e-13)
    np.testing.assert_allclose(var[1], delta ** 2 * (B * B - 1) / 12, rtol=1e-12)
    assert (var[2] == 0).all() and (mean[2] == 4.0).all()


def test_score_of_identical_keys_is_the_dot_product():
    rng = np.random.default_rng(0)
    k = rng.standard_normal(8)
    K = np.tile(k, (4, 1))
    q = rng.standard_normal(8)
    mean, var = O.block_statistics(K, 4)
    assert O.block_score(q, mean, var, 0.3)[0] == pytest.approx(0.3 * float(q @ k), rel=1e-14)


@pytest.mark.parametrize("seed", range(5))
def test_score_equals_block_average_of_second_order_expansion(seed):
    """For a block whose tokens each deviate from the mean along one channel
    (so the block covariance is diagonal), the average over its tokens of the
    second-order expansion of exp(sigma q.k) around the mean equals
    exp(score) exactly.  Computed token by token in plain Python."""
    rng = np.random.default_rng(seed)
    d, npairs = 6, 5
    mu = rng.standard_normal(d)
    toks = []
    for _ in range(npairs):
        c = int(rng.integers(d))
        dl = float(rng.uniform(0.2, 2.0))
        for sgn in (1, -1):
            t = mu.copy()
            t[c] += sgn * dl
            toks.append(t)
    K = np.array(toks)
    B = len(toks)
    q = rng.standard_normal(d)
    sigma = float(rng.uniform(0.1, 0.7))
    mean, var = O.block_statistics(K, B)
    score = O.block_score(q, mean, var, sigma)[0]
    a = sigma * sum(q[i] * mu[i] for i in range(d))
    avg = 0.0
    for t in toks:
        s = sigma * sum(q[i] * t[i] for i in range(d))
        avg += 1.0 + (s - a) + 0.5 * (s - a) ** 2
    avg /= B
    assert math.exp(score - a) == pytest.approx(avg, rel=1e-12)


# ----------------------------------------------------------------------------
# Candidates and selection
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("T,B,ns,Wn", [(100, 8, 4, 8), (100, 8, 0, 16), (64, 8, 8, 8), (20, 8, 4, 16),
                                       (33, 4, 9, 5), (5, 4, 4, 4), (129, 16, 20, 33)])
def test_candidates_match_token_level_definition(T, B, ns, Wn):
    p = _params(block_size=B, num_sink=ns, window=Wn)
    brute = sorted({t // B for t in range(T) if ns <= t < T - Wn})
    assert O.candidate_blocks(T, p).tolist() == brute
    for b in brute:                       # W >= B: every candidate is a full block
        assert (b + 1) * B <= T


@pytest.mark.parametrize("seed", range(6))
def test_top_k_matches_rank_count(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    cands = np.arange(n) + int(rng.integers(0, 3))
    scores = rng.choice(rng.standard_normal(max(1, n // 3)), size=n)   # many exact ties
    for k in [0, 1, 2, n // 2, n - 1, n, n + 3]:
        sel = O.select_top_k(cands, scores, k)
        want = []
        for i in range(n):
            better = sum(1 for j in range(n)
                         if scores[j] > scores[i] or (scores[j] == scores[i] and cands[j] < cands[i]))
            if better < k:
                want.append(int(cands[i]))
        assert sel.tolist() == want


def test_exact_and_residual_partition():
    rng = np.random.default_rng(3)
    for _ in range(20):
        B = int(rng.choice([2, 4, 8]))
        Wn = int(rng.integers(B, 4 * B))
        ns = int(rng.integers(0, 2 * B))
        T = int(rng.integers(1, 12 * B))
        p = _params(block_size=B, num_sink=ns, window=Wn)
        c = O.candidate_blocks(T, p)
        k = int(rng.integers(0, len(c) + 2))
        sel = c[rng.permutation(len(c))[:k]] if len(c) else c
        E = O.exact_token_mask(T, sel, p)
        assert E.sum() + (~E).sum() == T
        assert E[:min(ns, T)].all() and E[max(0, T - Wn):].all()
        covered = np.zeros(T, bool)
        for b in c:
            if b not in sel:
                covered[b * B:(b + 1) * B] = True
        assert not (~E & ~covered).any()          # U lies inside unselected candidates
        assert (not (~E).any()) == (k >= len(c))   # U empty iff every candidate is selected


# ----------------------------------------------------------------------------
# Whole decode: special cases, brute force, invariants
# ----------------------------------------------------------------------------

def _rand_case(rng, T, d, scale_k=1.0):
    K = rng.standard_normal((T, d)) * scale_k
    V = rng.standard_normal((T, d))
    q = rng.standard_normal(d)
    return q, K, V


def _sdpa(q, K, V, sigma, mask=None):
    qt = torch.from_numpy(q)[None, None, None, :]
    kt = torch.from_numpy(K)[None, None]
    vt = torch.from_numpy(V)[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=sigma)[0, 0, 0].numpy()


@pytest.mark.parametrize("form", ["definition", "subtraction"])
@pytest.mark.parametrize("T,B,ns,Wn,d", [(200, 8, 4, 16, 16), (97, 4, 0, 4, 8), (64, 16, 3, 16, 32), (10, 8, 4, 8, 4)])
def test_dense_when_budget_covers_all_candidates(form, T, B, ns, Wn, d):
    rng = np.random.default_rng(T + d)
    q, K, V = _rand_case(rng, T, d)
    p = _params(head_dim=d, block_size=B, num_sink=ns, window=Wn, top_k=10 ** 6)
    r = O.decode_head(q, K, V, p, form=form)
    assert r.exact.all() and r.den_u == 0.0
    np.testing.assert_allclose(r.out, _sdpa(q, K, V, p.sigma), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("d", [16, 64, 128])
def test_default_scale_is_the_standard_one(d):
    """With no scale given, the dense limit equals torch's attention at its
    own default scaling (1/sqrt(d)): pins the oracle's default sigma against
    a routine that fixes it independently."""
    rng = np.random.default_rng(d)
    q, K, V = _rand_case(rng, 120, d)
    p = _params(head_dim=d, block_size=8, num_sink=4, window=16, top_k=10 ** 6)
    assert p.scale == 0.0
    r = O.decode_head(q, K, V, p)
    qt, kt, vt = (torch.from_numpy(x)[None, None] for x in (q[None], K, V))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0, 0].numpy()
    np.testing.assert_allclose(r.out, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("form", ["definition", "subtraction"])
def test_sink_plus_window_when_no_budget_and_no_tail(form):
    rng = np.random.default_rng(11)
    T, d = 300, 16
    q, K, V = _rand_case(rng, T, d)
    p = _params(head_dim=d, block_size=8, num_sink=5, window=40, top_k=0, linear_tail=0)
    r = O.decode_head(q, K, V, p, form=form)
    mask = np.zeros(T, bool)
    mask[:5] = True
    mask[T - 40:] = True
    np.testing.assert_allclose(r.out, _sdpa(q, K, V, p.sigma, mask), rtol=1e-12, atol=1e-13)


def _brute_force(q, K, V, p):
    """Pure-Python per-token evaluation of the whole step on a tiny input."""
    T, d = len(K), len(q)
    B, sig = p.block_size, p.sigma
    Kl, Vl, ql = K.tolist(), V.tolist(), q.tolist()
    cands = [b for b in range(T // B) if any(p.num_sink <= t < T - p.window for t in range(b * B, (b + 1) * B))]
    sc = {}
    for b in cands:
        blk = Kl[b * B:(b + 1) * B]
        mu = [sum(t[c] for t in blk) / B for c in range(d)]
        va = [sum((t[c] - mu[c]) ** 2 for t in blk) / B for c in range(d)]
        sc[b] = sig * sum(ql[c] * mu[c] for c in range(d)) + math.log1p(
            0.5 * sig * sig * sum(ql[c] ** 2 * va[c] for c in range(d)))
    sel = [b for b in cands if sum(1 for o in cands if sc[o] > sc[b] or (sc[o] == sc[b] and o < b)) < p.top_k]
    num = [0.0] * d
    den = 0.0
    for t in range(T):
        s = sig * sum(ql[c] * Kl[t][c] for c in range(d))
        exact = t < p.num_sink or t >= T - p.window or (t // B) in sel
        if exact:
            w = math.exp(s)
        elif p.linear_tail:
            w = 1.0 + s
        else:
            continue
        den += w
        for c in range(d):
            num[c] += w * Vl[t][c]
    return np.array([x / den for x in num]), sel


@pytest.mark.parametrize("seed", range(8))
def test_against_per_token_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.choice([2, 4, 8]))
    d = int(rng.integers(1, 6))
    Wn = int(rng.integers(B, 3 * B))
    ns = int(rng.integers(0, B + 2))
    T = int(rng.integers(Wn + ns + 1, Wn + ns + 8 * B))
    k = int(rng.integers(0, 5))
    lt = int(rng.integers(0, 2))
    q, K, V = _rand_case(rng, T, d, scale_k=0.5)
    p = _params(head_dim=d, block_size=B, num_sink=ns, window=Wn, top_k=k, linear_tail=lt)
    want, sel = _brute_force(q, K, V, p)
    for form in ("definition", "subtraction"):
        r = O.decode_head(q, K, V, p, form=form)
        assert r.selected.tolist() == sel
        np.testing.assert_allclose(r.out, want, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_residual_state_equals_state_over_unselected_tokens(seed):
    rng = np.random.default_rng(200 + seed)
    T, d = 500, 12
    q, K, V = _rand_case(rng, T, d)
    p = _params(head_dim=d, block_size=16, num_sink=4, window=48, top_k=5)
    r_def = O.decode_head(q, K, V, p, form="definition")
    r_sub = O.decode_head(q, K, V, p, form="subtraction")
    G = O.global_state(K, V)
    E = r_sub.exact
    Ku, Vu = K[~E], V[~E]
    Su = O.state_over(K, V, ~E)
    # S_G minus the exact tokens' outer products equals the state built over U
    np.testing.assert_allclose(G.S - K[E].T @ V[E], Su.S, rtol=1e-12, atol=1e-11)
    np.testing.assert_allclose(G.z - K[E].sum(0), Su.z, rtol=1e-12, atol=1e-11)
    assert G.n - E.sum() == len(Ku) == Su.n
    np.testing.assert_allclose(r_sub.num_u, r_def.num_u, rtol=1e-10, atol=1e-10)
    assert r_sub.den_u == pytest.approx(r_def.den_u, rel=1e-12)
    np.testing.assert_allclose(r_sub.out, r_def.out, rtol=1e-12, atol=1e-13)


def test_linear_part_is_first_order_taylor_of_softmax():
    """Shrinking the query by eps, the hybrid output differs from dense
    softmax attention by O(eps^2): the linear weights 1 + s match exp(s) to
    first order (a sign or scale error in the kernel would leave O(eps))."""
    rng = np.random.default_rng(7)
    T, d = 400, 8
    q, K, V = _rand_case(rng, T, d)
    p = _params(head_dim=d, block_size=8, num_sink=2, window=16, top_k=3)
    errs = []
    for eps in (0.2, 0.1, 0.05):
        r = O.decode_head(eps * q, K, V, p)
        errs.append(np.abs(r.out - O.dense_attention(eps * q, K, V, p.sigma)).max())
    assert 3.3 < errs[0] / errs[1] < 4.7 and 3.3 < errs[1] / errs[2] < 4.7


def test_append_recurrence_matches_rebuild():
    rng = np.random.default_rng(9)
    d, B = 8, 8
    K = rng.standard_normal((77, d))
    V = rng.standard_normal((77, d))
    T0 = 50
    st = O.global_state(K[:T0], V[:T0])
    mean0, var0 = O.block_statistics(K[:T0], B)
    means, vars_ = list(mean0), list(var0)
    for t in range(T0, 77):
        st = O.append_token(st, K[t], V[t])
        fb = O.filled_block_stats(K[:t + 1], B)
        if fb is not None:
            b, mu, va = fb
            assert b == len(means)
            means.append(mu)
            vars_.append(va)
    full = O.global_state(K, V)
    np.testing.assert_allclose(st.S, full.S, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st.z, full.z, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st.sv, full.sv, rtol=1e-12, atol=1e-12)
    assert st.n == full.n
    m_full, v_full = O.block_statistics(K, B)
    np.testing.assert_allclose(np.array(means), m_full, rtol=1e-14)
    np.testing.assert_allclose(np.array(vars_), v_full, rtol=1e-13)


def test_needles_are_recalled():
    """Planted needle blocks (keys = 3 * unit query + noise) score far above
    the N(0,1) blocks, so every needle lands in its head's selection."""
    wl = W.small("needle_small")
    q = W.gen_queries(wl)
    p = O.Params(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, wl.top_k,
                 wl.num_sink, wl.window, wl.linear_tail)
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            K, V = W.gen_pair(wl, b, g, q)
            Kf, Vf = O.to_f64(K, wl.kv_dtype), O.to_f64(V, wl.kv_dtype)
            stats = O.block_statistics(Kf, wl.block_size)
            for blk, h in W.needle_plan(wl, b, g):
                r = O.decode_head(O.to_f64(q[b, h], wl.kv_dtype), Kf, Vf, p, stats=stats)
                assert blk in r.selected.tolist()


def test_generator_paging_round_trip():
    wl = W.small("ragged_small")
    inp = W.make_inputs(wl)
    for (b, g), (K, V) in inp["pairs"].items():
        np.testing.assert_array_equal(W.gather_pair(wl, inp["block_table"], inp["k_pages"], b, g), K)
        np.testing.assert_array_equal(W.gather_pair(wl, inp["block_table"], inp["v_pages"], b, g), V)
    used = set()
    for b in range(wl.batch):
        ids = inp["block_table"][b, :wl.blocks_mapped(b)].tolist()
        assert not used & set(ids)
        used |= set(ids)


# ----------------------------------------------------------------------------
# Grouped selection (one selection per kv head)
# ----------------------------------------------------------------------------

def test_golden_grouped_selection():
    ex = json.load(open(GOLDEN))["grouped_selection"]
    cands = np.array(ex["candidates"])
    c0 = ex["cases"][0]
    sc = np.array(c0["scores_num"])
    w = O.group_block_weights(sc)
    np.testing.assert_allclose(w * 20, c0["weights_over_20"], rtol=1e-14)
    for k, want in c0["selected"].items():
        assert O.select_top_k_grouped(cands, sc, int(k)).tolist() == want
    for h in range(2):   # the shared choice differs from each head's own top-1
        assert O.select_top_k(cands, sc[h], 1).tolist() == c0["per_head_top1"][h]
    c1 = ex["cases"][1]
    for k, want in c1["selected"].items():
        assert O.select_top_k_grouped(cands, np.array(c1["scores_num"]), int(k)).tolist() == want
    c2 = ex["cases"][2]   # the softmax shares, not the raw scores, are summed
    sc2 = np.array(c2["scores_num"], float)
    np.testing.assert_allclose(O.group_block_weights(sc2), c2["weights"], atol=1e-9)
    for k, want in c2["selected"].items():
        assert O.select_top_k_grouped(cands, sc2, int(k)).tolist() == want
    assert O.select_top_k(cands, sc2.sum(axis=0), 1).tolist() == c2["raw_sum_top1"]


@pytest.mark.parametrize("seed", range(6))
def test_grouped_with_one_head_is_the_per_head_selection(seed):
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(1, 80))
    cands = np.arange(n) + 1
    sc = rng.standard_normal(n) * 3
    for k in [0, 1, 5, n // 2, n, n + 2]:
        assert O.select_top_k_grouped(cands, sc[None, :], k).tolist() == O.select_top_k(cands, sc, k).tolist()


@pytest.mark.parametrize("seed", range(4))
def test_group_weights_sum_to_group_size_and_ignore_head_offsets(seed):
    rng = np.random.default_rng(400 + seed)
    G, n = int(rng.integers(2, 9)), int(rng.integers(2, 200))
    sc = rng.standard_normal((G, n)) * 4
    w = O.group_block_weights(sc)
    assert w.sum() == pytest.approx(G, rel=1e-12)
    assert (w > 0).all()
    shifted = sc + rng.standard_normal((G, 1)) * 50   # a constant per head
    np.testing.assert_allclose(O.group_block_weights(shifted), w, rtol=1e-9)


def test_identical_heads_select_as_one_head():
    rng = np.random.default_rng(7)
    p = _params(num_q_heads=4, num_kv_heads=1, head_dim=8, block_size=4, top_k=3, num_sink=2, window=8, grouped=1)
    K = rng.standard_normal((64, 8))
    q = rng.standard_normal(8)
    cands, scores, w, sel = O.group_selection(np.stack([q] * 4), K, p)
    assert sel.tolist() == O.select_top_k(cands, scores[0], p.top_k).tolist()


def test_grouped_batch_shares_the_selection_across_the_group():
    rng = np.random.default_rng(11)
    p = _params(num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=4, top_k=2, num_sink=1, window=8, grouped=1)
    T = 48
    pairs = {(0, g): (rng.standard_normal((T, 8)), rng.standard_normal((T, 8))) for g in range(2)}
    q = rng.standard_normal((1, 4, 8))
    res = O.decode_batch(q, pairs, p, [T])
    for g in range(2):
        sels = [res[(0, h)].selected.tolist() for h in (2 * g, 2 * g + 1)]
        assert sels[0] == sels[1]
        K, V = pairs[(0, g)]
        _, _, _, shared = O.group_selection(q[0, 2 * g:2 * g + 2], K, p)
        assert sels[0] == shared.tolist()
        for h in (2 * g, 2 * g + 1):   # each head decodes over the shared selection
            ref = O.decode_head(q[0, h], K, V, p, selected=shared)
            np.testing.assert_array_equal(res[(0, h)].out, ref.out)


def test_group_selection_scores_every_head_of_the_group():
    """The group's selection is the grouped top-k of the G heads' own block
    scores, as the per-head decode reports them."""
    rng = np.random.default_rng(19)
    G = 4
    p1 = _params(num_q_heads=G, num_kv_heads=1, head_dim=8, block_size=4, top_k=3, num_sink=1, window=8)
    pg = _params(num_q_heads=G, num_kv_heads=1, head_dim=8, block_size=4, top_k=3, num_sink=1, window=8, grouped=1)
    K, V = rng.standard_normal((80, 8)), rng.standard_normal((80, 8))
    qs = rng.standard_normal((G, 8)) * 2
    per_head = [O.decode_head(q, K, V, p1) for q in qs]
    want = O.select_top_k_grouped(per_head[0].candidates, np.stack([r.scores for r in per_head]), 3)
    cands, scores, w, sel = O.group_selection(qs, K, pg)
    assert sel.tolist() == want.tolist()
    np.testing.assert_array_equal(scores, np.stack([r.scores for r in per_head]))


# ----------------------------------------------------------------------------
# Token-level variant: top_k single tokens scored by their own keys
# ----------------------------------------------------------------------------

def _brute_force_tokens(q, K, V, p):
    """Pure-Python per-token evaluation of the token-level step on a tiny input:
    candidates [ns, T - W), score sigma q.k, top-k by rank counting."""
    T, d = len(K), len(q)
    sig = p.sigma
    Kl, Vl, ql = K.tolist(), V.tolist(), q.tolist()
    sc = {t: sig * sum(ql[c] * Kl[t][c] for c in range(d)) for t in range(p.num_sink, T - p.window)}
    sel = [t for t in sc if sum(1 for o in sc if sc[o] > sc[t] or (sc[o] == sc[t] and o < t)) < p.top_k]
    num = [0.0] * d
    den = 0.0
    for t in range(T):
        s = sig * sum(ql[c] * Kl[t][c] for c in range(d))
        if t < p.num_sink or t >= T - p.window or t in sel:
            w = math.exp(s)
        elif p.linear_tail:
            w = 1.0 + s
        else:
            continue
        den += w
        for c in range(d):
            num[c] += w * Vl[t][c]
    return np.array([x / den for x in num]), sel


@pytest.mark.parametrize("seed", range(8))
def test_token_level_against_per_token_brute_force(seed):
    rng = np.random.default_rng(700 + seed)
    B = int(rng.choice([2, 4, 8]))
    d = int(rng.integers(1, 6))
    Wn = int(rng.integers(B, 3 * B))
    ns = int(rng.integers(0, B + 2))
    T = int(rng.integers(Wn + ns + 1, Wn + ns + 40))
    k = int(rng.integers(0, 9))
    lt = int(rng.integers(0, 2))
    q, K, V = _rand_case(rng, T, d, scale_k=0.5)
    p = _params(head_dim=d, block_size=B, num_sink=ns, window=Wn, top_k=k, linear_tail=lt, tokens=1)
    want, sel = _brute_force_tokens(q, K, V, p)
    for form in ("definition", "subtraction"):
        r = O.decode_head(q, K, V, p, form=form)
        assert r.selected.tolist() == sel
        np.testing.assert_allclose(r.out, want, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_token_level_is_block_level_with_blocks_of_one_token(seed):
    """A one-token block has its key as mean and zero variance, so its block
    score is sigma q.k and its candidates are the tokens of [ns, T - W): the
    token-level step equals the block-level step at block size 1."""
    rng = np.random.default_rng(800 + seed)
    T, d = 300, 8
    q, K, V = _rand_case(rng, T, d)
    for k in (0, 7, 50):
        pt = _params(head_dim=d, block_size=16, num_sink=3, window=32, top_k=k, tokens=1)
        pb = _params(head_dim=d, block_size=1, num_sink=3, window=32, top_k=k)
        rt, rb = O.decode_head(q, K, V, pt), O.decode_head(q, K, V, pb)
        assert rt.selected.tolist() == rb.selected.tolist()
        assert (rt.exact == rb.exact).all()
        np.testing.assert_allclose(rt.out, rb.out, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("form", ["definition", "subtraction"])
def test_token_level_dense_when_budget_covers_all_candidates(form):
    rng = np.random.default_rng(901)
    T, d = 120, 8
    q, K, V = _rand_case(rng, T, d)
    p = _params(head_dim=d, block_size=8, num_sink=4, window=16, top_k=T, tokens=1)
    r = O.decode_head(q, K, V, p, form=form)
    assert r.exact.all() and r.den_u == 0.0
    np.testing.assert_allclose(r.out, _sdpa(q, K, V, p.sigma), rtol=1e-12, atol=1e-13)


def test_token_level_candidates_and_ties():
    p = _params(head_dim=2, block_size=4, num_sink=2, window=3, top_k=2, tokens=1)
    assert O.candidate_tokens(10, p).tolist() == [2, 3, 4, 5, 6]
    assert O.candidate_tokens(5, p).tolist() == []
    # equal scores go to the lower token index
    assert O.select_top_k(np.array([2, 3, 4, 5, 6]), np.array([0.5, 1.0, 1.0, 1.0, 0.2]), 2).tolist() == [3, 4]


# ----------------------------------------------------------------------------
# Multi-query (chunk) form: Q consecutive queries, each causal at its position
# ----------------------------------------------------------------------------

def _chunk_case(seed, T0, Q, d=8, B=4, **kw):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((T0 + Q, d))
    V = rng.standard_normal((T0 + Q, d))
    qc = rng.standard_normal((Q, d))
    p = _params(head_dim=d, block_size=B, **kw)
    return qc, K, V, p


@pytest.mark.parametrize("seed", [0, 1])
def test_chunk_all_exact_is_causal_dense_attention(seed):
    # budget covering every candidate: each query is plain softmax attention
    # over the tokens up to its own position; computed here as one masked
    # score matrix (rows = queries, columns = tokens) through torch
    T0, Q = 37, 6
    qc, K, V, p = _chunk_case(seed, T0, Q, top_k=64)
    rows = O.decode_chunk_head(qc, K, V, T0, p)
    q_t, k_t, v_t = (torch.from_numpy(x) for x in (qc, K, V))
    s = p.sigma * (q_t @ k_t.T)
    mask = torch.arange(T0 + Q)[None, :] <= (T0 + torch.arange(Q))[:, None]
    ref = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=1) @ v_t
    for i, r in enumerate(rows):
        np.testing.assert_allclose(r.out, ref[i].numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_chunk_rows_do_not_see_later_tokens(seed):
    # causality: row i is unchanged when every key and value after its
    # position is replaced; the rows after it change
    T0, Q = 45, 5
    qc, K, V, p = _chunk_case(seed, T0, Q, top_k=2, window=8)
    base = O.decode_chunk_head(qc, K, V, T0, p)
    for i in range(Q - 1):
        K2, V2 = K.copy(), V.copy()
        K2[T0 + i + 1:] += 3.0
        V2[T0 + i + 1:] -= 2.0
        alt = O.decode_chunk_head(qc, K2, V2, T0, p)
        for j in range(Q):
            if j <= i:
                np.testing.assert_array_equal(alt[j].out, base[j].out)
            else:
                assert not np.allclose(alt[j].out, base[j].out)


@pytest.mark.parametrize("seed", [0, 1])
def test_chunk_rows_against_per_token_brute_force(seed):
    # each row by direct per-token sums over its own exact and residual sets
    # (first-order Taylor weight 1 + s on the residual tokens), with the
    # chunk crossing a block boundary (T0 = 42, B = 4)
    T0, Q = 42, 6
    qc, K, V, p = _chunk_case(seed, T0, Q, top_k=2, window=8, num_sink=2)
    rows = O.decode_chunk_head(qc, K, V, T0, p)
    for i, r in enumerate(rows):
        L = T0 + i + 1
        assert r.exact[L - 1] and len(r.exact) == L          # the row's own token is exact
        num = np.zeros(K.shape[1])
        den = 0.0
        for t in range(L):
            st = p.sigma * float(K[t] @ qc[i])
            w = math.exp(st) if r.exact[t] else 1.0 + st
            num += w * V[t]
            den += w
        np.testing.assert_allclose(r.out, num / den, rtol=1e-11, atol=1e-12)
        # the window of row i starts at its own length minus W
        assert r.exact[L - p.window:].all()
