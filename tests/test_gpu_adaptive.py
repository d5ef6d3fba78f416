"""Parity of the adaptive-budget path (token coverage tau) with the oracle, through the C ABI.

Bars: the row budgets and the padded subsets bit-exact on the same fp32 scores (both
sides count the scores in 2^-40 units and decide with exact integer sums); gather and
scatter bit-exact on padded index lists; attention rows within 1e-4 (fp32) / 2e-2 (bf16);
the whole layer (fused bf16, staged fp32) end to end with unselected rows equal to the
residual bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._lib import ensure_built
from tests.gpu_helpers import TOL, check_adaptive_selection, dev, half_ulp, host, rel_err, round_to

pytestmark = pytest.mark.gpu

tsa = ensure_built()


def _scores(B, H, L, seed, kind):
    rng = np.random.default_rng(seed)
    if kind == "uniform":
        s = rng.random((B, H, L))
    elif kind == "ties":                       # few distinct values: long runs of equal scores
        s = np.round(rng.random((B, H, L)) * 16) / 16
    elif kind == "heavy":                      # a few positions hold most of the mass
        s = rng.pareto(1.2, (B, H, L)) * 1e-3
    elif kind == "tiny":                       # a third of the scores are below one 2^-40 unit
        s = rng.random((B, H, L))
        s[rng.random((B, H, L)) < 0.33] = 2.0 ** -45
    else:
        raise ValueError(kind)
    return s.astype(np.float32)


@pytest.mark.parametrize("B,H,L,keep,W,ns,kind,tau", [
    (1, 4, 1000, 1000, 16, 4, "uniform", 0.05),
    (2, 3, 777, 500, 5, 3, "ties", 0.2),       # the cap binds on some rows
    (1, 4, 5000, 5000, 64, 4, "heavy", 0.005),
    (1, 4, 5000, 2000, 64, 4, "heavy", 0.01),
    (1, 2, 300, 300, 64, 4, "tiny", 1e-9),     # only the zero-mass positions leave
    (1, 2, 300, 300, 64, 4, "uniform", 1.0),   # every candidate leaves: K = |F|
    (1, 2, 60, 60, 64, 4, "uniform", 0.5),     # no candidates at all
    (1, 1, 8, 8, 1, 1, "ties", 0.3),
    (1, 3, 131072, 131072, 64, 4, "heavy", 0.005),
    (1, 2, 131072, 65536, 64, 4, "ties", 0.3),
])
def test_budget_and_select_bitexact(B, H, L, keep, W, ns, kind, tau):
    s = _scores(B, H, L, L + H, kind)
    sg = torch.from_numpy(s).cuda()
    counts = tsa.budget(sg, keep, W, ns, tau=tau).cpu().numpy()
    want = oracle.coverage_budget(s, keep, W, ns, tau)
    print(f"{kind} tau={tau}: K/L {counts.min() / L:.3f} .. {counts.max() / L:.3f}")
    assert np.array_equal(counts, want)
    idx = tsa.select(sg, keep, W, ns, tau=tau).cpu().numpy()
    assert np.array_equal(idx, oracle.select(s, keep, W, ns, tau=tau))
    # the budget and the row lengths select writes agree
    assert np.array_equal((idx >= 0).sum(axis=-1), counts)


def test_budget_tau_zero_is_keep():
    s = _scores(2, 3, 500, 1, "uniform")
    counts = tsa.budget(torch.from_numpy(s).cuda(), 123, 8, 4).cpu().numpy()
    assert np.all(counts == 123)


@pytest.mark.parametrize("B,H,Hkv,L,keep,W,ns,kind,tau", [
    (1, 8, 2, 3000, 3000, 64, 4, "heavy", 0.01),
    (2, 4, 1, 999, 600, 7, 2, "ties", 0.25),
    (1, 32, 8, 131072, 131072, 64, 4, "uniform", 0.4),
])
def test_budget_and_select_per_kv_head_bitexact(B, H, Hkv, L, keep, W, ns, kind, tau):
    s = _scores(B, H, L, 7 + L, kind)
    sg = torch.from_numpy(s).cuda()
    counts = tsa.budget(sg, keep, W, ns, kv_heads=Hkv, tau=tau).cpu().numpy()
    assert np.array_equal(counts, oracle.coverage_budget(s, keep, W, ns, tau, kv_heads=Hkv))
    idx = tsa.select(sg, keep, W, ns, kv_heads=Hkv, tau=tau).cpu().numpy()
    assert np.array_equal(idx, oracle.select(s, keep, W, ns, Hkv, tau))


# ---- stages on padded index lists ---------------------------------------------------------

@pytest.mark.parametrize("dt,d,per_kv_head", [("bf16", 128, False), ("bf16", 128, True), ("fp32", 64, False)])
def test_stages_on_padded_idx(dt, d, per_kv_head):
    B, H, Hkv, L, keep, W, ns = 2, 8, 2, 700, 400, 16, 4
    x = workloads.small_random(B, H, Hkv, L, d, seed=31, dtype=dt)
    s = _scores(B, H, L, 3, "heavy")
    idx = oracle.select(s, keep, W, ns, Hkv if per_kv_head else None, 0.2 if per_kv_head else 0.05)
    ks = (idx >= 0).sum(axis=-1)
    assert ks.min() < keep and ks.max() > ks.min()
    q, k, v, r = (dev(x[n], dt) for n in "qkvr")
    ig = torch.from_numpy(idx.astype(np.int32)).cuda()
    qh, kh, vh = tsa.gather_qkv(q, k, v, ig)
    wq, wk, wv = oracle.gather(x["q"], x["k"], x["v"], idx)
    assert np.array_equal(host(qh), wq) and np.array_equal(host(kh), wk) and np.array_equal(host(vh), wv)
    oh = tsa.attn(qh, kh, vh)
    oh_or = oracle.attend(wq, wk, wv)
    err = float(np.max(np.abs(host(oh) - oh_or)))
    assert err <= TOL[dt], err
    # scatter of the GPU's attention rows: out-of-place and in place, bit-exact
    oh_vals = host(oh)
    want = round_to(oracle.scatter_residual(oh_vals, idx, x["r"]), dt)
    assert np.array_equal(host(tsa.scatter_residual(oh, ig, r)), want)
    r2 = r.clone()
    tsa.scatter_residual(oh, ig, r2, out=r2)
    assert np.array_equal(host(r2), want)


# ---- end to end -----------------------------------------------------------------------

def _end_to_end(x, dt, keep, W, ns, tau, in_place=False, per_kv_head=False, scale=0.0):
    q, k, v, r = (dev(x[n], dt) for n in "qkvr")
    Hkv = x["k"].shape[2]
    kvh = Hkv if per_kv_head else None
    if in_place:
        out = r.clone()
        _, sg, ig = tsa.forward(q, k, v, out, keep, W, ns, scale=scale, out=out, return_scores=True,
                                per_kv_head=per_kv_head, tau=tau)
    else:
        out, sg, ig = tsa.forward(q, k, v, r, keep, W, ns, scale=scale, return_scores=True,
                                  per_kv_head=per_kv_head, tau=tau)
    s32 = sg.cpu().numpy()
    idx = ig.cpu().numpy().astype(np.int64)
    d = x["q"].shape[-1]
    sc = scale if scale > 0 else 1.0 / np.sqrt(d)
    s64 = oracle.score(x["q"], x["k"], W, sc)
    assert rel_err(s32.astype(np.float64), s64) <= 1e-5
    # budgets and subsets bit-exact on the GPU's own scores
    assert np.array_equal(idx, oracle.select(s32, keep, W, ns, kvh, tau))
    # and valid under the coverage rule on the float64 scores (per KV head: their sums)
    n_tie = check_adaptive_selection(oracle.group_scores(s64, Hkv) if per_kv_head else s64, idx, keep, W, ns, tau)
    ks = (idx >= 0).sum(axis=-1)
    qh, kh, vh = oracle.gather(x["q"], x["k"], x["v"], idx)
    want = oracle.scatter_residual(oracle.attend(qh, kh, vh, sc), idx, x["r"])
    got = host(out)
    B, L, H, _ = x["q"].shape
    sel = np.zeros((B, L, H), dtype=bool)
    SG = H // idx.shape[1]
    for b in range(B):
        for h in range(H):
            row = idx[b, h // SG]
            sel[b, row[row >= 0], h] = True
    assert np.array_equal(got[~sel], x["r"][~sel].astype(np.float64))
    excess = np.abs(got[sel] - want[sel]) - half_ulp(got[sel], dt)
    print(f"adaptive {dt} tau={tau}{' per KV head' if per_kv_head else ''}: K {ks.min()}..{ks.max()} of cap "
          f"{keep}, near-tie differences from float64 {n_tie}, excess over half-ulp {excess.max():.3e}")
    assert excess.max() <= TOL[dt]
    return out, idx


@pytest.mark.parametrize("B,H,Hkv,L,d,keep,W,ns,tau,in_place,per_kv_head", [
    (1, 8, 2, 1500, 128, 1500, 64, 4, 0.2, False, False),
    (2, 8, 2, 1234, 128, 800, 32, 4, 0.1, False, False),     # the cap binds on some heads
    (1, 8, 2, 1500, 128, 1500, 64, 4, 0.3, True, False),
    (1, 8, 2, 1500, 128, 1500, 64, 4, 0.2, False, True),
    (1, 4, 4, 999, 64, 999, 16, 4, 0.5, False, False),
    (2, 8, 2, 1100, 128, 900, 64, 4, 0.25, True, True),       # per KV head, in place, B = 2
])
def test_forward_bf16_adaptive(B, H, Hkv, L, d, keep, W, ns, tau, in_place, per_kv_head):
    x = workloads.small_random(B, H, Hkv, L, d, seed=L + 11, dtype="bf16", q_grade=4.0)
    _end_to_end(x, "bf16", keep, W, ns, tau, in_place, per_kv_head)


@pytest.mark.parametrize("in_place,per_kv_head", [(False, False), (True, False), (False, True)])
def test_forward_fp32_adaptive(in_place, per_kv_head):
    x = workloads.small_random(1, 4, 2, 640, 64, seed=9, dtype="fp32", q_grade=3.0)
    _end_to_end(x, "fp32", 640, 32, 4, 0.25, in_place, per_kv_head)


@pytest.mark.parametrize("per_kv_head", [False, True])
def test_fused_adaptive_equals_staged(per_kv_head):
    # The fused forward runs only each subset's K_r rows; the staged path runs every compact
    # row, padding included.  Valid rows never see padded keys (causality), so the two
    # outputs agree bit for bit.
    B, H, Hkv, L, d, keep, W, ns, tau = 1, 8, 2, 2100, 128, 2100, 64, 4, 0.15
    x = workloads.small_random(B, H, Hkv, L, d, seed=77, dtype="bf16", q_grade=4.0)
    q, k, v, r = (dev(x[n], "bf16") for n in "qkvr")
    out, sg, ig = tsa.forward(q, k, v, r, keep, W, ns, return_scores=True, per_kv_head=per_kv_head, tau=tau)
    ks = (ig >= 0).sum(dim=-1)
    assert int(ks.min()) < int(ks.max())
    oh = tsa.attn(*tsa.gather_qkv(q, k, v, ig))
    staged = tsa.scatter_residual(oh, ig, r)
    assert torch.equal(out.view(torch.int16), staged.view(torch.int16))


def test_fused_adaptive_many_heads_without_plan():
    # More than 4096 (batch, head) pairs: the fused attention takes the interleaved tile
    # order instead of the per-XCD plan; it still equals the staged path bit for bit.
    B, H, Hkv, L, d, keep, W, ns, tau = 130, 32, 8, 200, 64, 200, 16, 4, 0.3
    x = workloads.small_random(B, H, Hkv, L, d, seed=5, dtype="bf16", q_grade=4.0)
    q, k, v, r = (dev(x[n], "bf16") for n in "qkvr")
    out, sg, ig = tsa.forward(q, k, v, r, keep, W, ns, return_scores=True, tau=tau)
    ks = (ig >= 0).sum(dim=-1)
    assert B * H > 4096 and int(ks.min()) < int(ks.max())
    assert np.array_equal(ig.cpu().numpy(), oracle.select(sg.cpu().numpy(), keep, W, ns, tau=tau))
    oh = tsa.attn(*tsa.gather_qkv(q, k, v, ig))
    staged = tsa.scatter_residual(oh, ig, r)
    assert torch.equal(out.view(torch.int16), staged.view(torch.int16))
