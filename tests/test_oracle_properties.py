"""Property tests of the float64 oracle on random tiny shapes (Hypothesis, derandomized so
every run draws the same cases).  Each property follows from the definitions the oracle
restates, independently of how it computes them:

* a subset holds exactly keep positions, ascending, every forced position among them, and
  no position left out beats a chosen one (higher score, or the same score and a lower
  position);
* every window row of the score is a probability distribution, so a head's scores sum to
  the number of window rows;
* keeping every position reproduces dense causal attention (torch SDPA in float64);
* positions outside every subset carry the residual unchanged;
* adaptive budgets lie between |F| and the cap, fall as tau grows, and what leaves fits
  the budget;
* drift lies in [0, 2] and is 0 for unchanged hidden states.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True)


@st.composite
def shapes(draw):
    Hkv = draw(st.integers(1, 2))
    G = draw(st.integers(1, 3))
    L = draw(st.integers(1, 40))
    W = draw(st.integers(1, 12))
    ns = draw(st.integers(0, 5))
    nF = len(oracle.forced_positions(L, W, ns))
    keep = draw(st.integers(nF, L))
    d = draw(st.sampled_from([4, 8]))
    B = draw(st.integers(1, 2))
    seed = draw(st.integers(0, 2 ** 16))
    return B, Hkv * G, Hkv, L, d, keep, W, ns, seed


def _inputs(B, H, Hkv, L, d, seed, ties=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, L, H, d))
    k = rng.standard_normal((B, L, Hkv, d))
    v = rng.standard_normal((B, L, Hkv, d))
    r = rng.standard_normal((B, L, H, d))
    if ties:
        q = np.round(q)
        k = np.round(k)
    return q, k, v, r


@SETTINGS
@given(shapes(), st.booleans())
def test_subset_structure_and_exchange(sh, ties):
    B, H, Hkv, L, d, keep, W, ns, seed = sh
    q, k, _, _ = _inputs(B, H, Hkv, L, d, seed, ties)
    s = oracle.score(q, k, W)
    idx = oracle.select(s, keep, W, ns)
    F_ = set(oracle.forced_positions(L, W, ns).tolist())
    for b in range(B):
        for h in range(H):
            row = idx[b, h].tolist()
            assert len(row) == keep and all(x < y for x, y in zip(row, row[1:]))
            assert F_ <= set(row)
            chosen = [p for p in row if p not in F_]
            left = [p for p in range(L) if p not in set(row)]
            for p in left:
                for c in chosen:
                    assert (s[b, h, c], -c) > (s[b, h, p], -p)


@SETTINGS
@given(shapes())
def test_score_rows_are_distributions(sh):
    B, H, Hkv, L, d, keep, W, ns, seed = sh
    q, k, _, _ = _inputs(B, H, Hkv, L, d, seed)
    s = oracle.score(q, k, W)
    assert np.all(s >= 0)
    np.testing.assert_allclose(s.sum(-1), min(W, L), rtol=1e-12)


@SETTINGS
@given(shapes())
def test_keep_all_is_dense_attention(sh):
    B, H, Hkv, L, d, keep, W, ns, seed = sh
    q, k, v, r = _inputs(B, H, Hkv, L, d, seed)
    out = oracle.forward(q, k, v, r, L, W, ns)["out"]
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3)))   # noqa: E731
    dense = F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True, enable_gqa=True)
    np.testing.assert_allclose(out, r + dense.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-10)


@SETTINGS
@given(shapes(), st.booleans())
def test_unselected_rows_keep_the_residual(sh, per_kv):
    B, H, Hkv, L, d, keep, W, ns, seed = sh
    q, k, v, r = _inputs(B, H, Hkv, L, d, seed)
    res = oracle.forward(q, k, v, r, keep, W, ns, per_kv_head=per_kv)
    idx = res["idx"]
    SG = H // idx.shape[1]
    for b in range(B):
        for h in range(H):
            others = np.setdiff1d(np.arange(L), idx[b, h // SG])
            assert np.array_equal(res["out"][b, others, h], r[b, others, h])


@SETTINGS
@given(shapes(), st.floats(1e-6, 1.0), st.floats(1e-6, 1.0))
def test_coverage_budget_bounds_and_monotone(sh, t1, t2):
    B, H, Hkv, L, d, keep, W, ns, seed = sh
    q, k, _, _ = _inputs(B, H, Hkv, L, d, seed)
    s = oracle.score(q, k, W).astype(np.float32)
    lo, hi = sorted((t1, t2))
    nF = len(oracle.forced_positions(L, W, ns))
    k_lo = oracle.coverage_budget(s, keep, W, ns, lo)
    k_hi = oracle.coverage_budget(s, keep, W, ns, hi)
    assert np.all((nF <= k_hi) & (k_hi <= k_lo) & (k_lo <= keep))
    idx = oracle.select(s, keep, W, ns, tau=hi)
    for b in range(B):
        for h in range(H):
            units = oracle.mass_units(s[b, h])
            budget = math.floor(float(np.float32(hi)) * float(sum(units)))
            kept = set(idx[b, h][idx[b, h] >= 0].tolist())
            left = [p for p in range(L) if p not in kept]
            if k_hi[b, h] < keep:                     # the rule, not the cap, decided
                assert sum(units[p] for p in left) <= budget


@SETTINGS
@given(st.integers(1, 30), st.integers(1, 16), st.integers(0, 2 ** 16))
def test_drift_range(n, dim, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((1, n, dim))
    b = rng.standard_normal((1, n, dim))
    assert -1e-12 <= oracle.drift(a, b) <= 2 + 1e-12
    assert abs(oracle.drift(a, a)) < 1e-12
