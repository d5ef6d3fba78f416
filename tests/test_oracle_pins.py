"""Pins of the float64 oracle to things other than itself (CPU only).

Each test ties one oracle stage to what the pages and the mathematics fix:
hand-worked exact cases, a closed form, a library routine (torch's scaled dot-product
attention in float64, which also fixes the grouped-query head map), brute force on tiny
inputs, and invariants of the definition.  Together they are chosen so that a dropped
scale, a non-causal mask, a wrong window, a wrong KV head, a wrong tie order, a
score-ordered subset, a missing sink or a residual added in the wrong places fails at
least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _num(x):
    if isinstance(x, str):
        if x == "sqrt2ln2":
            return math.sqrt(2.0) * math.log(2.0)
        return float(Fraction(x))
    return float(x)


def _arr(rows):
    return np.array([[_num(c) for c in row] for row in rows], dtype=np.float64)


def _hand_inputs(case):
    g = json.load(open(GOLDEN))
    c, e = g["common"], g[case]
    L, d = c["L"], c["d"]
    q = np.zeros((1, L, 1, d))
    k = np.zeros((1, L, 1, d))
    for p, row in e["q_nonzero"].items():
        q[0, int(p), 0] = [_num(x) for x in row]
    for p, row in e["k_nonzero"].items():
        k[0, int(p), 0] = [_num(x) for x in row]
    v = _arr(c["v"]).reshape(1, L, 1, d)
    r = _arr(c["r"]).reshape(1, L, 1, d)
    return c, e, q, k, v, r


@pytest.mark.parametrize("case", ["case1", "case2"])
def test_hand_cases_exact(case):
    c, e, q, k, v, r = _hand_inputs(case)
    res = oracle.forward(q, k, v, r, keep=c["keep"], W=c["W"], n_sink=c["n_sink"])
    np.testing.assert_allclose(res["scores"][0, 0], [_num(x) for x in e["scores"]], rtol=0, atol=1e-15)
    assert res["idx"][0, 0].tolist() == e["idx"]
    np.testing.assert_allclose(res["oh"][0, 0], _arr(e["oh"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(res["out"][0, :, 0], _arr(e["out"]), rtol=0, atol=1e-14)


def _harmonic(n):
    return sum(1.0 / m for m in range(1, n + 1))


@pytest.mark.parametrize("L,W,n_sink,keep", [(64, 8, 4, 20), (50, 50, 0, 50), (33, 1, 3, 10)])
def test_zero_query_closed_form(L, W, n_sink, keep):
    # q = 0: row i spreads weight 1/(i+1) over keys 0..i, so s_j = H_L - H_{max(j, L-W')}.
    rng = np.random.default_rng(1)
    d = 4
    q = np.zeros((1, L, 2, d))
    k = rng.standard_normal((1, L, 1, d))
    s = oracle.score(q, k, W)
    Wp = min(W, L)
    want = np.array([_harmonic(L) - _harmonic(max(j, L - Wp)) for j in range(L)])
    np.testing.assert_allclose(s[0, 0], want, rtol=0, atol=1e-13)
    np.testing.assert_allclose(s[0, 1], want, rtol=0, atol=1e-13)
    # Every key before the window ties, so the lowest positions fill the budget.
    idx = oracle.select(s, keep, W, n_sink)
    expect = sorted(set(range(keep - Wp)) | set(range(L - Wp, L)))
    assert idx[0, 0].tolist() == expect


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x))


def _sdpa(q_blhd, k_blhd, v_blhd, scale=None):
    """torch SDPA (float64, CPU, causal, grouped-query) on [B,L,H,d] tensors -> [B,L,H,dv]."""
    qt = _t(q_blhd).permute(0, 2, 1, 3)
    kt = _t(k_blhd).permute(0, 2, 1, 3)
    vt = _t(v_blhd).permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, enable_gqa=True, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("B,H,Hkv,L,d", [(2, 4, 2, 37, 16), (1, 8, 2, 64, 8), (1, 3, 3, 9, 5)])
def test_keep_all_equals_dense_sdpa(B, H, Hkv, L, d):
    # keep = L: S_h = [0, L), so Out - R is plain causal attention ("sparse equals dense").
    x = workloads.small_random(B, H, Hkv, L, d, seed=7)
    res = oracle.forward(x["q"], x["k"], x["v"], x["r"], keep=L, W=3, n_sink=2)
    assert all((res["idx"][b, h] == np.arange(L)).all() for b in range(B) for h in range(H))
    want = _sdpa(x["q"].astype(np.float64), x["k"].astype(np.float64), x["v"].astype(np.float64))
    np.testing.assert_allclose(res["out"] - x["r"], want, rtol=0, atol=1e-12)


def test_attend_matches_sdpa_on_subset():
    x = workloads.small_random(1, 4, 2, 60, 16, seed=3)
    res = oracle.forward(x["q"], x["k"], x["v"], x["r"], keep=21, W=4, n_sink=2)
    # SDPA on the compact tensors ([B,H,keep,d] -> [B,keep,H,d] view).
    qh, kh, vh = (np.transpose(t, (0, 2, 1, 3)) for t in (res["qh"], res["kh"], res["vh"]))
    want = _sdpa(qh, kh, vh)
    np.testing.assert_allclose(np.transpose(res["oh"], (0, 2, 1, 3)), want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("B,H,Hkv,L,d,W", [(1, 4, 2, 24, 8, 5), (2, 6, 3, 17, 4, 17), (1, 2, 1, 12, 6, 40)])
def test_score_matches_sdpa_probabilities(B, H, Hkv, L, d, W):
    # With V = identity (one-hot value rows), SDPA returns the causal probability rows
    # themselves; the score is their sum over the last W' rows.
    x = workloads.small_random(B, H, Hkv, L, d, seed=11)
    eye = np.broadcast_to(np.eye(L)[None, :, None, :], (B, L, Hkv, L)).copy()
    P = _sdpa(x["q"].astype(np.float64), x["k"].astype(np.float64), eye)   # [B, L(query), H, L(key)]
    Wp = min(W, L)
    want = P[:, L - Wp:, :, :].sum(axis=1)                                  # [B, H, L]
    s = oracle.score(x["q"], x["k"], W)
    np.testing.assert_allclose(s, want, rtol=0, atol=1e-13)
    np.testing.assert_allclose(s.sum(axis=-1), Wp, rtol=0, atol=1e-12)   # each row's weights sum to 1


def _check_subset(s_row, S, keep, W, n_sink):
    L = len(s_row)
    S = list(S)
    assert len(S) == keep
    assert all(a < b for a, b in zip(S, S[1:]))
    Fset = set(range(min(n_sink, L))) | set(range(L - min(W, L), L))
    assert Fset <= set(S)
    chosen = [c for c in S if c not in Fset]
    unchosen = [u for u in range(L) if u not in set(S)]
    for c in chosen:            # brute-force exchange property of top-k with ties to the lower position
        for u in unchosen:
            assert s_row[c] > s_row[u] or (s_row[c] == s_row[u] and c < u)


@pytest.mark.parametrize("seed", range(8))
def test_select_exchange_property(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(6, 40))
    W = int(rng.integers(1, 6))
    n_sink = int(rng.integers(0, 5))
    nF = len(oracle.forced_positions(L, W, n_sink))
    keep = int(rng.integers(nF, L + 1))
    s = np.round(rng.random(L) * 4) / 4          # few distinct values: many ties
    s[:n_sink] = 0.0                              # sinks score lowest but must stay
    S = oracle.select_row(s, keep, W, n_sink)
    _check_subset(s, S, keep, W, n_sink)


def test_select_edge_cases():
    s = np.linspace(1.0, 0.0, 10)
    assert oracle.select_row(s, 10, 3, 2).tolist() == list(range(10))            # keep = L
    assert oracle.select_row(s, 5, 3, 2).tolist() == [0, 1, 7, 8, 9]            # keep = |F|
    assert oracle.select_row(s, 10, 64, 4).tolist() == list(range(10))          # W >= L: everything forced
    assert oracle.select_row(s, 4, 2, 2).tolist() == [0, 1, 8, 9]
    assert oracle.select_row(np.zeros(6), 6, 2, 8).tolist() == list(range(6))    # sinks beyond L clip
    with pytest.raises(ValueError):
        oracle.select_row(s, 4, 3, 2)                                            # keep < |F|
    with pytest.raises(ValueError):
        oracle.select_row(s, 11, 3, 2)                                           # keep > L


def test_threshold_hand_case():
    # L = 10, W = 2, one sink: F = {0, 8, 9}, and the forced positions score highest, so a
    # threshold that counted them would come out too high.  The candidates 1..7 score
    # 5, 3, 5, 1, 5, 0, 2, so the taken scores in order are 5, 5, 5, 3, 2, 1, 0.
    s = np.array([9.0, 5.0, 3.0, 5.0, 1.0, 5.0, 0.0, 2.0, 7.0, 8.0])
    assert oracle.threshold(s, 3, 2, 1) == math.inf           # keep = |F|: no candidate taken
    assert oracle.threshold(s, 4, 2, 1) == 5.0                # first of three tied 5s
    assert oracle.threshold(s, 6, 2, 1) == 5.0                # last of the tied 5s
    assert oracle.threshold(s, 7, 2, 1) == 3.0
    assert oracle.threshold(s, 9, 2, 1) == 1.0
    assert oracle.threshold(s, 10, 2, 1) == 0.0               # keep = L: the lowest candidate
    # The threshold is the lowest score among the non-forced positions the select takes.
    for keep in range(4, 11):
        S = oracle.select_row(s, keep, 2, 1)
        taken = [p for p in S if p not in (0, 8, 9)]
        assert oracle.threshold(s, keep, 2, 1) == min(s[taken])


@pytest.mark.parametrize("seed", range(12))
def test_threshold_brute_force(seed):
    # Brute force by counting: theta is the largest candidate score t such that at least
    # keep - |F| candidates score t or more (no sort, no select involved).
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(5, 30))
    W = int(rng.integers(1, 5))
    n_sink = int(rng.integers(0, 4))
    F = set(oracle.forced_positions(L, W, n_sink).tolist())
    cand = [p for p in range(L) if p not in F]
    s = np.round(rng.random(L) * 6) / 6                        # many ties
    for p in F:
        s[p] = 2.0 + rng.random()                              # forced positions score above every candidate
    for keep in range(len(F), L + 1):
        n = keep - len(F)
        if n == 0:
            want = math.inf
        else:
            want = max(t for t in (s[p] for p in cand) if sum(s[u] >= t for u in cand) >= n)
        assert oracle.threshold(s, keep, W, n_sink) == want, (keep, n)


def test_gather_scatter_brute_force():
    x = workloads.small_random(2, 4, 2, 9, 3, seed=5)
    idx = np.array([[[0, 2, 5, 8], [1, 2, 3, 8], [0, 4, 7, 8], [3, 5, 6, 8]]] * 2)
    qh, kh, vh = oracle.gather(x["q"], x["k"], x["v"], idx)
    oh = np.random.default_rng(0).standard_normal(qh.shape)
    out = oracle.scatter_residual(oh, idx, x["r"])
    for b in range(2):
        for h in range(4):
            for t in range(4):
                p = int(idx[b, h, t])
                for c in range(3):
                    assert qh[b, h, t, c] == x["q"][b, p, h, c]
                    assert kh[b, h, t, c] == x["k"][b, p, h // 2, c]
                    assert vh[b, h, t, c] == x["v"][b, p, h // 2, c]
            for p in range(9):
                for c in range(3):
                    want = float(x["r"][b, p, h, c])
                    if p in idx[b, h].tolist():
                        want += oh[b, h, idx[b, h].tolist().index(p), c]
                    assert out[b, p, h, c] == want


def test_attention_special_values():
    rng = np.random.default_rng(2)
    n, d = 17, 6
    qh = rng.standard_normal((1, 1, n, d))
    vh = rng.standard_normal((1, 1, n, d))
    # K^ = 0: uniform causal weights, a running mean of V^.
    oh = oracle.attend(qh, np.zeros_like(qh), vh)
    want = np.cumsum(vh[0, 0], axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(oh[0, 0], want, rtol=0, atol=1e-14)
    # V^ constant: any convex combination returns it.
    c = rng.standard_normal(d)
    oh = oracle.attend(qh, rng.standard_normal((1, 1, n, d)), np.broadcast_to(c, (1, 1, n, d)))
    np.testing.assert_allclose(oh[0, 0], np.broadcast_to(c, (n, d)), rtol=0, atol=1e-14)


def test_unselected_rows_equal_residual_bitwise():
    x = workloads.small_random(1, 4, 2, 40, 8, seed=9, dtype="bf16")
    res = oracle.forward(x["q"], x["k"], x["v"], x["r"], keep=12, W=4, n_sink=2)
    for h in range(4):
        mask = np.ones(40, dtype=bool)
        mask[res["idx"][0, h]] = False
        assert np.array_equal(res["out"][0, mask, h], x["r"][0, mask, h].astype(np.float64))
        assert not np.array_equal(res["out"][0, ~mask, h], x["r"][0, ~mask, h].astype(np.float64))


def test_attend_rows_matches_attend():
    x = workloads.small_random(1, 2, 1, 30, 8, seed=4)
    res = oracle.forward(x["q"], x["k"], x["v"], x["r"], keep=14, W=3, n_sink=1)
    rows = [0, 5, 13]
    o = oracle.attend_rows(res["qh"][0, 1], res["kh"][0, 1], res["vh"][0, 1], rows, 1 / np.sqrt(8))
    np.testing.assert_allclose(o, res["oh"][0, 1, rows], rtol=0, atol=1e-15)


def test_planted_tokens_recovered_small():
    # A reduced planted workload: every planted key should be selected by every head
    # of its KV group (the planted keys align with the window queries).
    w = workloads.WORKLOADS["bf16_L64k_planted"].with_(B=1, L=4096, keep=409)
    x = workloads.make_inputs(w)
    s = oracle.score(x["q"], x["k"], w.W)
    idx = oracle.select(s, w.keep, w.W, w.n_sink)
    for g in range(w.Hkv):
        P = set(x["planted"][(0, g)].tolist())
        for h in range(g * w.G, (g + 1) * w.G):
            assert len(P & set(idx[0, h].tolist())) == len(P)


def test_inputs_reproducible_and_bf16_exact():
    a = workloads.small_random(1, 2, 1, 5000, 4, seed=3, dtype="bf16")
    b = workloads.small_random(1, 2, 1, 5000, 4, seed=3, dtype="bf16")
    assert np.array_equal(a["q"], b["q"]) and np.array_equal(a["r"], b["r"])
    assert np.array_equal(workloads.round_bf16(a["k"]), a["k"])
    t = torch.from_numpy(np.ascontiguousarray(a["v"])).to(torch.bfloat16).float().numpy()
    assert np.array_equal(t, a["v"])          # bf16-exact values survive torch's conversion
    raw = np.random.default_rng(0).standard_normal(1000, dtype=np.float32)
    want = torch.from_numpy(raw).to(torch.bfloat16).float().numpy()
    assert np.array_equal(workloads.round_bf16(raw), want)   # our RNE equals torch's


# ---- subsets per KV head (an extension of the library: the pages define per-head subsets) ----

def test_group_select_hand_case():
    # Query heads 0 and 1 share KV head 0; L = 8, one sink and a window of one: F = {0, 7}.
    # Worked by hand: the summed row is [0, 5, 5, 4, 4, 0, 0, 0].  keep 4 takes the two
    # fives (positions 1, 2); keep 5 also takes one of the tied fours, the lower (3).  Per
    # head the subsets differ: head 0 takes 1 (5) and 4 (2), head 1 takes 2 and 3 (4, 4).
    s = np.zeros((1, 2, 8))
    s[0, 0] = [0, 5, 1, 0, 2, 0, 0, 0]
    s[0, 1] = [0, 0, 4, 4, 2, 0, 0, 0]
    assert oracle.select(s, 4, 1, 1, kv_heads=1).tolist() == [[[0, 1, 2, 7]]]
    assert oracle.select(s, 5, 1, 1, kv_heads=1).tolist() == [[[0, 1, 2, 3, 7]]]
    assert oracle.select(s, 4, 1, 1).tolist() == [[[0, 1, 4, 7], [0, 2, 3, 7]]]


def test_group_select_identical_heads_and_g1():
    rng = np.random.default_rng(11)
    base = np.round(rng.random((2, 3, 40)) * 8) / 4            # quarter steps: sums stay exact, many ties
    s = np.repeat(base, 4, axis=1)                              # 3 KV heads x 4 identical query heads
    shared = oracle.select(s, 20, 5, 4, kv_heads=3)
    per_head = oracle.select(base, 20, 5, 4)
    assert np.array_equal(shared, per_head)
    # one query head per KV head: the shared rule is the per-head rule
    assert np.array_equal(oracle.select(base, 20, 5, 4, kv_heads=3), per_head)


@pytest.mark.parametrize("seed", range(4))
def test_group_select_exchange_property(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(8, 40))
    W = int(rng.integers(1, 6))
    n_sink = int(rng.integers(0, 5))
    nF = len(oracle.forced_positions(L, W, n_sink))
    keep = int(rng.integers(nF, L + 1))
    s = np.round(rng.random((1, 4, L)) * 4) / 4                 # 2 KV heads x 2 query heads, ties
    idx = oracle.select(s, keep, W, n_sink, kv_heads=2)
    for g in range(2):
        summed = s[0, 2 * g] + s[0, 2 * g + 1]                  # exact in quarter steps
        _check_subset(summed, idx[0, g], keep, W, n_sink)


def test_group_gather_scatter_brute_force():
    x = workloads.small_random(2, 4, 2, 9, 3, seed=7)            # G = 2: subsets r = h // 2
    idx = np.array([[[0, 2, 5, 8], [1, 2, 3, 8]], [[0, 4, 7, 8], [3, 5, 6, 8]]])
    qh, kh, vh = oracle.gather(x["q"], x["k"], x["v"], idx)
    assert qh.shape == (2, 4, 4, 3) and kh.shape == (2, 2, 4, 3)
    oh = np.random.default_rng(1).standard_normal(qh.shape)
    out = oracle.scatter_residual(oh, idx, x["r"])
    for b in range(2):
        for h in range(4):
            sub = idx[b, h // 2].tolist()
            for t in range(4):
                for c in range(3):
                    assert qh[b, h, t, c] == x["q"][b, sub[t], h, c]
                    assert kh[b, h // 2, t, c] == x["k"][b, sub[t], h // 2, c]
                    assert vh[b, h // 2, t, c] == x["v"][b, sub[t], h // 2, c]
            for p in range(9):
                for c in range(3):
                    want = float(x["r"][b, p, h, c])
                    if p in sub:
                        want += oh[b, h, sub.index(p), c]
                    assert out[b, p, h, c] == want


def test_group_attend_equals_repeated_rows():
    rng = np.random.default_rng(4)
    qh = rng.standard_normal((1, 4, 30, 8))
    kh = rng.standard_normal((1, 2, 30, 8))
    vh = rng.standard_normal((1, 2, 30, 8))
    shared = oracle.attend(qh, kh, vh)
    repeated = oracle.attend(qh, np.repeat(kh, 2, axis=1), np.repeat(vh, 2, axis=1))   # per-head form, pinned by SDPA
    assert np.array_equal(shared, repeated)


def test_group_forward_equals_per_head_when_queries_coincide():
    # If the query heads of a KV head carry the same queries, their scores coincide, so the
    # shared subset is each head's own subset and the whole layer agrees with per-head mode.
    x = workloads.small_random(1, 4, 2, 48, 8, seed=9)
    q = x["q"].copy()
    q[:, :, 1] = q[:, :, 0]
    q[:, :, 3] = q[:, :, 2]
    a = oracle.forward(q, x["k"], x["v"], x["r"], 20, 6, 2, per_kv_head=True)
    b = oracle.forward(q, x["k"], x["v"], x["r"], 20, 6, 2)
    assert np.array_equal(a["idx"][:, [0, 0, 1, 1]], b["idx"])
    assert np.array_equal(a["out"], b["out"])


# ---- adaptive budgets (token coverage tau) --------------------------------------------
# The rule is this library's reading of the paper page's token coverage (TL;DR, Figures 1
# and 5): lowest-scoring non-forced positions leave while their summed score stays within
# tau times the row's total; masses are counted in 2^-40 units.

def test_mass_units_exact():
    assert oracle.mass_units([0.5, 2.0 ** -40, 2.0 ** -41, 3.0, 0.0]) == [2 ** 39, 1, 0, 3 * 2 ** 40, 0]
    x = float(np.float32(0.1))                    # not dyadic-short: rounds down
    assert oracle.mass_units([x])[0] == int(Fraction(x) * 2 ** 40)


def test_coverage_hand_case():
    # L=12, W=2, one sink: forced {0, 10, 11}.  Total 16.8125; tau=0.1 (float32 0.100000001..)
    # gives a budget just above 1.68125.  Leaving order (score up, then position down):
    # 6 (.0625) 8 (.125) 3 (.125) 4 (.25) 1 (.25) 9 (.5) 2 (.5) 5 (1) 7 (2); cumulative
    # .0625 .1875 .3125 .5625 .8125 1.3125 | 1.8125 > budget, so six leave and 2 (tied with
    # 9) stays: K = 6, S = {0, 2, 5, 7, 10, 11}.
    s = np.array([[[5, 0.25, 0.5, 0.125, 0.25, 1, 0.0625, 2, 0.125, 0.5, 3, 4]]], dtype=np.float64)
    assert oracle.coverage_budget(s, 12, 2, 1, 0.1).tolist() == [[6]]
    assert oracle.select(s, 12, 2, 1, tau=0.1)[0, 0].tolist() == [0, 2, 5, 7, 10, 11] + [-1] * 6
    # the cap: at most keep positions
    assert oracle.select(s, 5, 2, 1, tau=0.1)[0, 0].tolist() == [0, 5, 7, 10, 11]
    # six leave once the budget reaches 1.3125, five just below it
    assert oracle.coverage_budget_row(s[0, 0], 12, 2, 1, 0.0781) == 6     # budget 1.31306
    assert oracle.coverage_budget_row(s[0, 0], 12, 2, 1, 0.078) == 7      # budget 1.31138


@pytest.mark.parametrize("seed", range(6))
def test_coverage_brute_force_max_leavers(seed):
    # The number of positions that leave is the largest number of non-forced positions
    # whose unit masses fit in the budget (exhaustive over subsets), and the kept set is
    # the top-K set of the fixed-budget rule.
    rng = np.random.default_rng(seed)
    L, W, ns = 10, 2, 1
    s = np.round(rng.random(L) * 8) / 8 + rng.integers(0, 2, L) * rng.random(L)
    units = oracle.mass_units(s)
    F = set(oracle.forced_positions(L, W, ns).tolist())
    cand = [j for j in range(L) if j not in F]
    for tau in (0.0001, 0.02, 0.1, 0.3, 0.7, 1.0):
        budget = math.floor(float(np.float32(tau)) * float(sum(units)))
        best = 0
        for mask in range(1 << len(cand)):
            members = [cand[i] for i in range(len(cand)) if mask >> i & 1]
            if sum(units[j] for j in members) <= budget:
                best = max(best, len(members))
        k = oracle.coverage_budget_row(s, L, W, ns, tau)
        assert k == L - best, (tau, k, best)
        row = oracle.select(s[None, None], L, W, ns, tau=tau)[0, 0]
        assert row[:k].tolist() == oracle.select_row(s, k, W, ns).tolist()
        assert (row[k:] == -1).all()
        dropped = sorted(set(range(L)) - set(row[:k].tolist()))
        assert sum(units[j] for j in dropped) <= budget


def test_coverage_limits_and_monotone():
    rng = np.random.default_rng(3)
    L, W, ns = 200, 8, 4
    s = rng.random(L) + 2.0 ** -30                 # every score at least one unit
    assert oracle.coverage_budget_row(s, L, W, ns, 1e-30) == L            # budget 0: nobody leaves
    assert oracle.coverage_budget_row(s, L, W, ns, 1.0) == ns + W         # everything non-forced leaves
    ks = [oracle.coverage_budget_row(s, L, W, ns, t) for t in (1e-6, 1e-4, 1e-3, 0.01, 0.05, 0.2, 0.5, 0.9)]
    assert all(a >= b for a, b in zip(ks, ks[1:])) and ks[0] > ks[-1]
    # zero-mass positions (below one unit) leave even with a zero budget
    z = s.copy()
    z[[20, 30, 40]] = 2.0 ** -45
    assert oracle.coverage_budget_row(z, L, W, ns, 1e-30) == L - 3


def test_coverage_uniform_closed_form():
    # All candidates score x: floor(budget / units(x)) of them leave (at most all of them).
    L, W, ns = 100, 4, 2
    for x, tau in ((0.75, 0.05), (0.3, 0.013), (1.0, 0.5)):
        s = np.full(L, x)
        u = oracle.mass_units([x])[0]
        budget = math.floor(float(np.float32(tau)) * float(u * L))
        n_cand = L - ns - W
        assert oracle.coverage_budget_row(s, L, W, ns, tau) == L - min(n_cand, budget // u)
        # ties leave from the highest position down: the kept candidates are the lowest ones
        k = oracle.coverage_budget_row(s, L, W, ns, tau)
        row = oracle.select(s[None, None], L, W, ns, tau=tau)[0, 0, :k]
        assert row.tolist() == list(range(k - W)) + list(range(L - W, L))


def test_coverage_group_rows_and_padding_through_stages():
    # Per KV head the budget is taken on the summed rows; padded idx entries give zero
    # gathered rows and are skipped by the scatter, and valid compact rows never see them.
    x = workloads.small_random(1, 4, 2, 40, 8, seed=5, dtype="f32")
    s = oracle.score(x["q"], x["k"], 8).astype(np.float32)
    kv = oracle.coverage_budget(s, 40, 8, 2, 0.05, kv_heads=2)
    gs = oracle.group_scores(s, 2)
    assert kv.tolist() == [[oracle.coverage_budget_row(gs[0, g], 40, 8, 2, 0.05) for g in range(2)]]
    idx = oracle.select(s, 30, 8, 2, tau=0.3)
    qh, kh, vh = oracle.gather(x["q"], x["k"], x["v"], idx)
    oh = oracle.attend(qh, kh, vh)
    out = oracle.scatter_residual(oh, idx, x["r"])
    ks = (idx[0] >= 0).sum(axis=1)
    assert ks.min() < 30                           # the rule binds below the cap somewhere
    for h in range(4):
        k_h = int(ks[h])
        assert np.all(qh[0, h, k_h:] == 0) and np.all(kh[0, h, k_h:] == 0)
        sub = oracle.attend(qh[:, h:h + 1, :k_h], kh[:, h:h + 1, :k_h], vh[:, h:h + 1, :k_h])
        np.testing.assert_allclose(oh[0, h, :k_h], sub[0, 0], rtol=1e-12, atol=1e-12)
        rows = idx[0, h, :k_h]
        others = np.setdiff1d(np.arange(40), rows)
        assert np.array_equal(out[0, others, h], np.asarray(x["r"], dtype=np.float64)[0, others, h])
        np.testing.assert_allclose(out[0, rows, h], x["r"][0, rows, h] + oh[0, h, :k_h], rtol=1e-12, atol=1e-12)


# ---- representation drift (skill page, Step 4) -----------------------------------------

def test_drift_closed_forms():
    rng = np.random.default_rng(8)
    a = rng.standard_normal((3, 50, 64))
    assert abs(oracle.drift(a, a)) < 1e-15                       # unchanged: cosine 1
    assert abs(oracle.drift(a, 3.5 * a)) < 1e-15                 # positive rescaling does not count
    assert abs(oracle.drift(a, -a) - 2.0) < 1e-15                # reversed: cosine -1
    # orthogonal pairs: swap the two halves of a vector with one sign flipped
    b = np.concatenate([-a[..., 32:], a[..., :32]], axis=-1)
    assert abs(oracle.drift(a, b) - 1.0) < 1e-14
    # hand case: cosines 0, 1 and 1/2 (a 60 degree angle) -> drift 1 - 1/2 = 0.5
    h0 = np.array([[1.0, 0.0], [1.0, 1.0], [1.0, 0.0]])
    h1 = np.array([[0.0, 2.0], [3.0, 3.0], [1.0, math.sqrt(3.0)]])
    assert abs(oracle.drift(h0, h1) - 0.5) < 1e-15
    # a zero vector is normalised to zero (the norm is clamped at 1e-12): its cosine is 0
    z = np.zeros((2, 4))
    z[1] = [1, 2, 3, 4]
    assert abs(oracle.drift(z, np.ones((2, 4))) - (1 - (0 + 10 / (math.sqrt(30) * 2)) / 2)) < 1e-15
    # tokens are weighted equally whatever their norms
    big = np.array([[1000.0, 0.0], [0.0, 0.001]])
    assert abs(oracle.drift(big, np.array([[1.0, 0.0], [1.0, 0.0]])) - 0.5) < 1e-15


def test_drift_small_angle_and_torch_cosine():
    # Against torch's own cosine_similarity (float64, with its eps far below these norms).
    rng = np.random.default_rng(9)
    a = rng.standard_normal((2, 30, 128))
    b = a + 0.05 * rng.standard_normal(a.shape)
    cos = F.cosine_similarity(torch.from_numpy(a), torch.from_numpy(b), dim=-1).numpy()
    assert abs(oracle.drift(a, b) - (1.0 - cos.mean())) < 1e-14
    assert 0 < oracle.drift(a, b) < 0.01


def test_layer_stable_window_rule():
    # not before three drifts; then the mean of the last three against 0.1
    assert oracle.layer_stable([0.0, 0.0]) == [False, False]
    d = [0.05, 0.05, 0.05, 0.3, 0.01, 0.01, 0.01, 0.1, 0.1, 0.1]
    assert oracle.layer_stable(d) == [False, False, True, False, False, False, True, True, True, False]
    assert oracle.layer_stable([0.2, 0.0, 0.05], window=2, threshold=0.1) == [False, False, True]
