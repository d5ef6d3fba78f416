"""Parity at the full workload sizes, through tsa_forward as bench.py calls it.

The oracle cannot redo a whole 131072-token layer in seconds, so each case checks what
it can compute one by one: the scores, subset and attention rows of a sample of heads
(exact oracle arithmetic on those heads), and, over the whole tensor, the properties
that hold at any size (unselected rows equal the residual bit for bit; every subset has
keep ascending positions including the forced ones).  The planted-importance workload
also checks that every head of a KV group keeps that group's planted keys and that the
heads' subsets differ."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._lib import ensure_built
from tests.gpu_helpers import TOL, check_adaptive_selection, check_selection, half_ulp, rel_err

pytestmark = pytest.mark.gpu

tsa = ensure_built()

_CACHE = {}


def _inputs(name):
    w = workloads.WORKLOADS[name]
    key = (w.B, w.L, w.H, w.Hkv, w.d, w.dtype, w.planted, w.seed, w.q_grade)
    if key not in _CACHE:
        _CACHE.clear()
        _CACHE[key] = workloads.make_inputs(w)
    return w, _CACHE[key]


def _run(w, x):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v, r = (torch.from_numpy(x[n]).to(dt).cuda() for n in "qkvr")
    out, sg, ig = tsa.forward(q, k, v, r, w.keep, w.W, w.n_sink, return_scores=True)
    torch.cuda.synchronize()
    return q, k, v, r, out, sg, ig


def _check(w, x, heads, rows_per_head=12, seed=0):
    q, k, v, r, out, sg, ig = _run(w, x)
    B, L, H, d = x["q"].shape
    G = H // w.Hkv
    scale = 1.0 / np.sqrt(d)

    # Whole-tensor properties.
    idx_all = ig.cpu().numpy().astype(np.int64)
    assert idx_all.shape == (B, H, w.keep)
    assert np.all(np.diff(idx_all, axis=-1) > 0)
    F = oracle.forced_positions(L, w.W, w.n_sink)
    assert np.all(np.isin(F, idx_all[0, 0])) and np.all(np.isin(F, idx_all[-1, -1]))
    sel = torch.zeros(B, H, L, dtype=torch.bool, device="cuda")
    sel.scatter_(2, ig.long(), True)
    sel = sel.permute(0, 2, 1)                                  # [B, L, H]
    assert torch.equal(out[~sel].view(torch.int16), r[~sel].view(torch.int16))
    assert int(sel.sum()) == B * H * w.keep

    rng = np.random.default_rng(seed)
    s_gpu_all = sg.cpu().numpy().astype(np.float64)
    worst_s, worst_out, n_diff = 0.0, 0.0, 0
    for b, h in heads:
        g = h // G
        qh = x["q"][b, :, h, :].astype(np.float64)
        kg = x["k"][b, :, g, :].astype(np.float64)
        vg = x["v"][b, :, g, :].astype(np.float64)
        s_or = oracle.score_head(qh, kg, w.W, scale)
        s_gpu = s_gpu_all[b, h]
        worst_s = max(worst_s, rel_err(s_gpu, s_or))
        idx = idx_all[b, h]
        assert np.array_equal(idx, oracle.select_row(s_gpu, w.keep, w.W, w.n_sink))   # select bit-exact
        n_diff += check_selection(s_or[None, None], idx[None, None], w.keep, w.W, w.n_sink)
        # Attention rows on the GPU's subset: first, last and random compact rows.
        rows = np.unique(np.concatenate([[0, w.keep - 1], rng.integers(0, w.keep, rows_per_head)]))
        o_rows = oracle.attend_rows(qh[idx], kg[idx], vg[idx], rows, scale)
        pos = idx[rows]
        got = out[b, torch.from_numpy(pos).cuda(), h, :].float().cpu().numpy().astype(np.float64)
        want = x["r"][b, pos, h, :].astype(np.float64) + o_rows
        excess = np.abs(got - want) - half_ulp(got, w.dtype)
        worst_out = max(worst_out, float(excess.max()))
    print(f"{w.name}: score rel err {worst_s:.2e}, out excess {worst_out:.2e}, subset differences {n_diff}")
    assert worst_s <= 1e-5
    assert worst_out <= TOL[w.dtype]
    return idx_all


def test_full_bf16_L8k_r05():
    w, x = _inputs("bf16_L8k_r0.5")
    _check(w, x, heads=[(0, 0), (0, 5), (0, 13), (0, 31)])


def test_full_bf16_L32k_r025():
    w, x = _inputs("bf16_L32k_r0.25")
    _check(w, x, heads=[(0, 2), (0, 19)])


@pytest.mark.parametrize("name", ["bf16_L128k_r0.1", "bf16_L128k_r0.25", "bf16_L128k_r0.5"])
def test_full_bf16_L128k(name):
    w, x = _inputs(name)
    _check(w, x, heads=[(0, 0), (0, 30)], rows_per_head=8)


def test_full_planted_recall_and_distinct_heads():
    w, x = _inputs("bf16_L64k_planted")
    idx = _check(w, x, heads=[(0, 1), (1, 22)], rows_per_head=8)
    G = w.G
    recalls, jac = [], []
    for b in range(w.B):
        for g in range(w.Hkv):
            P = x["planted"][(b, g)]
            sets = []
            for h in range(g * G, (g + 1) * G):
                S = idx[b, h]
                recalls.append(np.isin(P, S).mean())
                sets.append(set(S.tolist()))
            for i in range(G):
                for j in range(i + 1, G):
                    assert sets[i] != sets[j]
                    jac.append(len(sets[i] & sets[j]) / len(sets[i] | sets[j]))
    print(f"planted recall min {min(recalls):.4f} mean {np.mean(recalls):.4f}; within-group Jaccard mean "
          f"{np.mean(jac):.3f} max {max(jac):.3f}")
    assert min(recalls) >= 0.99
    assert max(jac) < 0.5


def test_full_per_kv_head_L128k():
    # Subsets shared per KV head at L = 131072, keep 0.25, through tsa_forward (bf16 fused).
    w, x = _inputs("bf16_L128k_r0.25")
    dt = torch.bfloat16
    q, k, v, r = (torch.from_numpy(x[n]).to(dt).cuda() for n in "qkvr")
    out, sg, ig = tsa.forward(q, k, v, r, w.keep, w.W, w.n_sink, return_scores=True, per_kv_head=True)
    torch.cuda.synchronize()
    B, L, H, d = x["q"].shape
    G = H // w.Hkv
    scale = 1.0 / np.sqrt(d)
    idx_all = ig.cpu().numpy().astype(np.int64)
    assert idx_all.shape == (B, w.Hkv, w.keep)
    assert np.all(np.diff(idx_all, axis=-1) > 0)
    F = oracle.forced_positions(L, w.W, w.n_sink)
    assert all(np.all(np.isin(F, idx_all[b, g])) for b in range(B) for g in range(w.Hkv))
    sel = torch.zeros(B, w.Hkv, L, dtype=torch.bool, device="cuda")
    sel.scatter_(2, ig.long(), True)
    sel = sel.repeat_interleave(G, dim=1).permute(0, 2, 1)       # [B, L, H]: head h uses subset h // G
    assert torch.equal(out[~sel].view(torch.int16), r[~sel].view(torch.int16))
    s32 = sg.cpu().numpy()
    rng = np.random.default_rng(2)
    worst_s, worst_out, n_diff = 0.0, 0.0, 0
    for b, g in [(0, 1), (0, 6)]:
        heads = range(g * G, (g + 1) * G)
        kg = x["k"][b, :, g, :].astype(np.float64)
        vg = x["v"][b, :, g, :].astype(np.float64)
        s_or = np.stack([oracle.score_head(x["q"][b, :, h, :].astype(np.float64), kg, w.W, scale) for h in heads])
        worst_s = max(worst_s, rel_err(s32[b, g * G:(g + 1) * G].astype(np.float64), s_or))
        idx = idx_all[b, g]
        # select bit-exact on the GPU's own fp32 scores, summed in fp32 in ascending head order
        assert np.array_equal(idx, oracle.select(s32[b:b + 1, g * G:(g + 1) * G], w.keep, w.W, w.n_sink,
                                                 kv_heads=1)[0, 0])
        n_diff += check_selection(oracle.group_scores(s_or[None], 1), idx[None, None], w.keep, w.W, w.n_sink)
        for h in (heads[0], heads[-1]):
            qh = x["q"][b, :, h, :].astype(np.float64)
            rows = np.unique(np.concatenate([[0, w.keep - 1], rng.integers(0, w.keep, 6)]))
            o_rows = oracle.attend_rows(qh[idx], kg[idx], vg[idx], rows, scale)
            pos = idx[rows]
            got = out[b, torch.from_numpy(pos).cuda(), h, :].float().cpu().numpy().astype(np.float64)
            want = x["r"][b, pos, h, :].astype(np.float64) + o_rows
            worst_out = max(worst_out, float((np.abs(got - want) - half_ulp(got, w.dtype)).max()))
    print(f"{w.name} per KV head: score rel err {worst_s:.2e}, out excess {worst_out:.2e}, "
          f"subset differences {n_diff}")
    assert worst_s <= 1e-5
    assert worst_out <= TOL[w.dtype]


def test_full_adaptive_graded_L128k():
    # Adaptive budgets (token coverage 0.2, no cap below L) at L = 131072 through
    # tsa_forward (bf16 fused), heads graded from diffuse to concentrated attention.
    w, x = _inputs("bf16_L128k_tau0.2_graded")
    dt = torch.bfloat16
    q, k, v, r = (torch.from_numpy(x[n]).to(dt).cuda() for n in "qkvr")
    out, sg, ig = tsa.forward(q, k, v, r, w.keep, w.W, w.n_sink, return_scores=True, tau=w.tau)
    torch.cuda.synchronize()
    B, L, H, d = x["q"].shape
    G = H // w.Hkv
    scale = 1.0 / np.sqrt(d)
    s32 = sg.cpu().numpy()
    idx_all = ig.cpu().numpy().astype(np.int64)
    # budgets and subsets of every head bit-exact on the GPU's own scores
    assert np.array_equal(idx_all, oracle.select(s32, w.keep, w.W, w.n_sink, tau=w.tau))
    # and valid under the coverage rule on float64 scores, on heads from diffuse to sharp
    heads = [0, 10, 21, 31]
    s_or = np.stack([oracle.score_head(x["q"][0, :, h, :].astype(np.float64), x["k"][0, :, h // G, :].astype(np.float64),
                                       w.W, scale) for h in heads])[None]
    n_tie = check_adaptive_selection(s_or, idx_all[:, heads], w.keep, w.W, w.n_sink, w.tau)
    print(f"{w.name}: near-tie differences from float64 scores on heads {heads}: {n_tie}")
    ks = (idx_all >= 0).sum(axis=-1)
    print(f"{w.name}: K/L per head {ks.min() / L:.3f} .. {ks.max() / L:.3f}, mean {ks.mean() / L:.3f}")
    assert ks[0, 0] > ks[0, -1]                    # sharper heads keep fewer positions
    sel = torch.zeros(B, H, L + 1, dtype=torch.bool, device="cuda")
    sel.scatter_(2, torch.where(ig >= 0, ig, L).long(), True)
    sel = sel[:, :, :L].permute(0, 2, 1)
    assert torch.equal(out[~sel].view(torch.int16), r[~sel].view(torch.int16))
    assert int(sel.sum()) == int(ks.sum())
    rng = np.random.default_rng(4)
    worst_s, worst_out = 0.0, 0.0
    for b, h in [(0, 0), (0, 31)]:
        g = h // G
        qh = x["q"][b, :, h, :].astype(np.float64)
        kg = x["k"][b, :, g, :].astype(np.float64)
        vg = x["v"][b, :, g, :].astype(np.float64)
        worst_s = max(worst_s, rel_err(s32[b, h].astype(np.float64), oracle.score_head(qh, kg, w.W, scale)))
        kh_ = int(ks[b, h])
        idx = idx_all[b, h, :kh_]
        rows = np.unique(np.concatenate([[0, kh_ - 1], rng.integers(0, kh_, 8)]))
        o_rows = oracle.attend_rows(qh[idx], kg[idx], vg[idx], rows, scale)
        pos = idx[rows]
        got = out[b, torch.from_numpy(pos).cuda(), h, :].float().cpu().numpy().astype(np.float64)
        want = x["r"][b, pos, h, :].astype(np.float64) + o_rows
        worst_out = max(worst_out, float((np.abs(got - want) - half_ulp(got, w.dtype)).max()))
    print(f"{w.name}: score rel err {worst_s:.2e}, out excess {worst_out:.2e}")
    assert worst_s <= 1e-5
    assert worst_out <= TOL[w.dtype]


@pytest.mark.parametrize("name", ["bf16_L32k_r0.25", "bf16_L128k_r0.5"])
def test_full_dense_attention_sampled_rows(name):
    # The library's dense causal attention (the denominator of every speedup figure) at
    # L = 32768 and L = 131072: sampled rows of sampled heads against the oracle's
    # attention with every position kept (keep = L: the subset is the whole sequence).
    w, x = _inputs(name)
    q, k, v = (torch.from_numpy(x[n]).to(torch.bfloat16).cuda() for n in "qkv")
    o = tsa.dense_attn(q, k, v)
    torch.cuda.synchronize()
    B, L, H, d = x["q"].shape
    G = H // w.Hkv
    scale = 1.0 / np.sqrt(d)
    rng = np.random.default_rng(11)
    worst = 0.0
    for b, h in [(0, 0), (0, 13), (0, 31)]:
        rows = np.unique(np.concatenate([[0, 1, 63, 64, L - 1], rng.integers(0, L, 6)]))
        want = oracle.attend_rows(x["q"][b, :, h, :], x["k"][b, :, h // G, :], x["v"][b, :, h // G, :], rows, scale)
        got = o[b, torch.from_numpy(rows).cuda(), h, :].float().cpu().numpy().astype(np.float64)
        worst = max(worst, float(np.max(np.abs(got - want))))
    print(f"{name} dense attention: max abs err {worst:.2e} on sampled rows")
    assert worst <= TOL["bf16"]


def test_full_compact_attention_n65536():
    # tsa_attn on the compact rows of the L = 131072 keep 0.5 layer (n = 65536 rows per
    # head): sampled rows of two heads against the oracle on the same subsets.
    w, x = _inputs("bf16_L128k_r0.5")
    q, k, v, r = (torch.from_numpy(x[n]).to(torch.bfloat16).cuda() for n in "qkvr")
    _, _, ig = tsa.forward(q, k, v, r, w.keep, w.W, w.n_sink, return_scores=True)
    oh = tsa.attn(*tsa.gather_qkv(q, k, v, ig))
    torch.cuda.synchronize()
    idx_all = ig.cpu().numpy().astype(np.int64)
    d = w.d
    scale = 1.0 / np.sqrt(d)
    rng = np.random.default_rng(12)
    worst = 0.0
    for b, h in [(0, 4), (0, 27)]:
        g = h // w.G
        idx = idx_all[b, h]
        rows = np.unique(np.concatenate([[0, 383, 384, w.keep - 1], rng.integers(0, w.keep, 6)]))
        want = oracle.attend_rows(x["q"][b, idx, h, :], x["k"][b, idx, g, :], x["v"][b, idx, g, :], rows, scale)
        got = oh[b, h, torch.from_numpy(rows).cuda(), :].float().cpu().numpy().astype(np.float64)
        worst = max(worst, float(np.max(np.abs(got - want))))
    print(f"compact attention n = {w.keep}: max abs err {worst:.2e} on sampled rows")
    assert worst <= TOL["bf16"]


def test_full_sparse_attn_in_place_equals_forward():
    # The launch the benchmark times for the attention roofline: tsa_sparse_attn in place
    # on the subsets tsa_forward chose (one fused attention kernel) writes what the forward
    # wrote, over the whole L = 131072 tensor.
    w, x = _inputs("bf16_L128k_r0.5")
    q, k, v, r = (torch.from_numpy(x[n]).to(torch.bfloat16).cuda() for n in "qkvr")
    out, _, ig = tsa.forward(q, k, v, r, w.keep, w.W, w.n_sink, return_scores=True)
    r2 = r.clone()
    tsa.sparse_attn(q, k, v, ig, r2, out=r2)
    torch.cuda.synchronize()
    assert torch.equal(r2, out)


def test_full_graded_fixed_budget_selection():
    # Sharp logits (query scale up to 4 on the graded workload) with a fixed budget of half
    # the positions: the GPU subsets may differ from the subsets of the float64 oracle
    # scores only at near-ties (relative gap 1e-6), checked on the sharpest, a middle and
    # the most diffuse head.
    w, x = _inputs("bf16_L128k_tau0.2_graded")
    keep = w.L // 2
    q, k, v, r = (torch.from_numpy(x[n]).to(torch.bfloat16).cuda() for n in "qkvr")
    _, sg, ig = tsa.forward(q, k, v, r, keep, w.W, w.n_sink, return_scores=True)
    torch.cuda.synchronize()
    s_gpu = sg.cpu().numpy().astype(np.float64)
    idx_all = ig.cpu().numpy().astype(np.int64)
    scale = 1.0 / np.sqrt(w.d)
    worst_s, n_diff = 0.0, 0
    for h in (31, 16, 0):
        g = h // w.G
        s_or = oracle.score_head(x["q"][0, :, h, :].astype(np.float64), x["k"][0, :, g, :].astype(np.float64),
                                 w.W, scale)
        worst_s = max(worst_s, rel_err(s_gpu[0, h], s_or))
        assert np.array_equal(idx_all[0, h], oracle.select_row(s_gpu[0, h], keep, w.W, w.n_sink))
        n_diff += check_selection(s_or[None, None], idx_all[0, h][None, None], keep, w.W, w.n_sink)
    print(f"graded fixed budget keep {keep}: score rel err {worst_s:.2e}, subset differences {n_diff}")
