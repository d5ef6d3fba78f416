"""Parity of the HIP path (through the C ABI) with the float64 oracle, stage by stage and
end to end, at sizes the oracle finishes in seconds, spanning several tiles and ragged
tails.  Bars: bit-exact for select, gather and scatter; max abs error 1e-4 (fp32) or
2e-2 (bf16) for attention; scores within a relative 1e-5 of the oracle (the selection
rule allows set differences only at near-ties of relative gap 1e-6)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._lib import ensure_built
from tests.gpu_helpers import TOL, check_selection, dev, half_ulp, host, rel_err, round_to

pytestmark = pytest.mark.gpu

tsa = ensure_built()


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    maps = open("/proc/self/maps").read()
    hip = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    print("HIP runtimes loaded:", hip, flush=True)


# ---- select: bit-exact on the same fp32 scores ------------------------------------------

@pytest.mark.parametrize("B,H,L,keep,W,ns,ties", [
    (1, 4, 512, 256, 32, 4, False),
    (2, 3, 1000, 137, 5, 3, False),
    (1, 2, 1000, 137, 5, 3, True),
    (1, 2, 777, 68, 64, 4, False),          # keep = |F|: nothing chosen
    (1, 2, 777, 777, 64, 4, False),         # keep = L: everything
    (1, 2, 40, 40, 64, 4, False),           # window covers the sequence
    (1, 1, 8, 3, 1, 1, True),
    (1, 3, 131072, 13107, 64, 4, False),
    (1, 2, 131072, 65536, 64, 4, True),
    (1, 1, 70000, 5000, 17, 9, True),
    # rows up to 16384 run the one-workgroup select (2, 4, 8 and 16 positions per thread);
    # 16385 is the shortest row of the multi-workgroup path
    (1, 2, 2000, 700, 16, 2, True),
    (1, 3, 3500, 1000, 64, 4, True),
    (2, 2, 5000, 1300, 64, 4, False),
    (1, 2, 9000, 4500, 64, 4, True),
    (1, 3, 16384, 4096, 64, 4, False),
    (1, 2, 16384, 10000, 64, 4, True),
    (1, 2, 16385, 4096, 64, 4, True),
    (1, 3, 32768, 8192, 64, 4, False),
])
def test_select_bitexact(B, H, L, keep, W, ns, ties):
    rng = np.random.default_rng(L + keep)
    s = rng.random((B, H, L)).astype(np.float32) * 0.01
    if ties:
        s = np.round(s * 200) / 200          # few distinct values: long runs of equal scores
        s = s.astype(np.float32)
    s[..., :ns] = 0.0
    sg = torch.from_numpy(s).cuda()
    idx = tsa.select(sg, keep, W, ns).cpu().numpy()
    want = oracle.select(s.astype(np.float64), keep, W, ns)
    assert np.array_equal(idx, want)


# ---- gather / scatter: bit-exact ------------------------------------------------------

@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 64), ("fp32", 64), ("fp32", 128)])
def test_gather_scatter_bitexact(dt, d):
    B, H, Hkv, L, keep = 2, 8, 2, 300, 77
    x = workloads.small_random(B, H, Hkv, L, d, seed=21, dtype=dt)
    rng = np.random.default_rng(5)
    idx = np.stack([np.stack([np.sort(rng.choice(L, keep, replace=False)) for _ in range(H)]) for _ in range(B)])
    q, k, v, r = (dev(x[n], dt) for n in "qkvr")
    ig = torch.from_numpy(idx.astype(np.int32)).cuda()
    qh, kh, vh = tsa.gather_qkv(q, k, v, ig)
    wq, wk, wv = oracle.gather(x["q"], x["k"], x["v"], idx)
    assert np.array_equal(host(qh), wq) and np.array_equal(host(kh), wk) and np.array_equal(host(vh), wv)

    oh_vals = rng.standard_normal((B, H, keep, d)).astype(np.float32)
    oh_vals = workloads.round_bf16(oh_vals) if dt == "bf16" else oh_vals
    oh = dev(oh_vals, dt)
    want = round_to(oracle.scatter_residual(oh_vals, idx, x["r"]), dt)
    out = tsa.scatter_residual(oh, ig, r)
    assert np.array_equal(host(out), want)
    r2 = r.clone()
    tsa.scatter_residual(oh, ig, r2, out=r2)      # in place
    assert np.array_equal(host(r2), want)


# ---- attention on compact rows and dense -------------------------------------------------

@pytest.mark.parametrize("dt,d,n", [("bf16", 128, 1), ("bf16", 128, 31), ("bf16", 128, 300), ("bf16", 128, 1000),
                                    # bf16: a wave holds 48 query rows, a workgroup 384
                                    ("bf16", 128, 47), ("bf16", 128, 48), ("bf16", 128, 385), ("bf16", 128, 769),
                                    ("bf16", 64, 384), ("bf16", 64, 515),
                                    ("fp32", 64, 256), ("fp32", 64, 700), ("fp32", 128, 333)])
def test_attn_compact(dt, d, n):
    B, H = 2, 3
    rng = np.random.default_rng(n + d)
    qh, kh, vh = (rng.standard_normal((B, H, n, d)).astype(np.float32) for _ in range(3))
    if dt == "bf16":
        qh, kh, vh = (workloads.round_bf16(t) for t in (qh, kh, vh))
    oh = tsa.attn(dev(qh, dt), dev(kh, dt), dev(vh, dt))
    want = oracle.attend(qh, kh, vh)
    err = np.max(np.abs(host(oh) - want))
    print(f"attn {dt} d={d} n={n}: max abs err {err:.3e}")
    assert err <= TOL[dt]


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 64), ("fp32", 128)])
def test_attn_logit_jumps(dt, d):
    # Keys aligned with every query at a few late positions make a row's logits jump by
    # more than 32 in log2 units mid-row (the running softmax reference must move and O
    # be rescaled there), and an early huge logit makes every later probability tiny.
    B, H, n = 1, 2, 700
    rng = np.random.default_rng(11 + d)
    u = np.ones(d) / np.sqrt(d)
    qh = rng.standard_normal((B, H, n, d)) * 0.3 + 8.0 * u
    kh = rng.standard_normal((B, H, n, d)) * 0.3
    vh = rng.standard_normal((B, H, n, d))
    kh[:, 0, 5] = 60.0 * u                     # head 0: early dominant key
    for pos, b in ((150, 40.0), (400, 80.0), (650, 120.0)):
        kh[:, 1, pos] = b * u                  # head 1: jumps of ~40 log2 units each
    qh, kh, vh = (t.astype(np.float32) for t in (qh, kh, vh))
    if dt == "bf16":
        qh, kh, vh = (workloads.round_bf16(t) for t in (qh, kh, vh))
    oh = tsa.attn(dev(qh, dt), dev(kh, dt), dev(vh, dt))
    want = oracle.attend(qh, kh, vh)
    err = np.max(np.abs(host(oh) - want))
    print(f"attn jumps {dt} d={d}: max abs err {err:.3e}")
    assert err <= TOL[dt]


@pytest.mark.parametrize("dt,d,H,Hkv,L", [("bf16", 128, 8, 2, 777), ("bf16", 128, 4, 4, 200), ("fp32", 64, 4, 1, 390)])
def test_dense_attn(dt, d, H, Hkv, L):
    x = workloads.small_random(1, H, Hkv, L, d, seed=8, dtype=dt)
    o = tsa.dense_attn(dev(x["q"], dt), dev(x["k"], dt), dev(x["v"], dt))
    res = oracle.forward(x["q"], x["k"], x["v"], np.zeros_like(x["r"]), keep=L, W=1, n_sink=0)
    err = np.max(np.abs(host(o) - res["out"]))
    print(f"dense {dt} L={L}: max abs err {err:.3e}")
    assert err <= TOL[dt]


def test_compact_with_keep_all_equals_dense():
    # keep = L on the compact path must reproduce the dense kernel bit for bit.
    x = workloads.small_random(1, 4, 2, 500, 128, seed=2, dtype="bf16")
    q, k, v = (dev(x[n], "bf16") for n in "qkv")
    dense = tsa.dense_attn(q, k, v)
    idx = torch.arange(500, dtype=torch.int32, device="cuda").repeat(1, 4, 1).contiguous()
    qh, kh, vh = tsa.gather_qkv(q, k, v, idx)
    oh = tsa.attn(qh, kh, vh)
    assert torch.equal(oh.permute(0, 2, 1, 3), dense)


# ---- scoring ------------------------------------------------------------------------------

@pytest.mark.parametrize("dt,d,B,H,Hkv,L,W", [("bf16", 128, 1, 8, 2, 1000, 64), ("bf16", 128, 2, 4, 4, 333, 5),
                                              ("bf16", 64, 1, 4, 1, 2048, 32), ("fp32", 64, 1, 4, 4, 512, 32),
                                              ("fp32", 128, 1, 2, 1, 97, 64), ("bf16", 128, 1, 2, 2, 40, 64),
                                              ("fp32", 64, 1, 2, 2, 77, 1),
                                              # bf16 head groups: two quads (G = 8), partial quads (G = 2, 3),
                                              # d = 64 with 64 window rows, many chunks with a ragged end, L = 1
                                              ("bf16", 128, 1, 16, 2, 1500, 64), ("bf16", 128, 2, 6, 2, 700, 40),
                                              ("bf16", 64, 1, 4, 2, 3001, 64), ("bf16", 128, 1, 2, 1, 20000, 64),
                                              ("bf16", 128, 1, 4, 1, 1, 64),
                                              # d = 64 with one and three 16-row window blocks
                                              ("bf16", 64, 1, 4, 2, 1000, 16), ("bf16", 64, 2, 8, 2, 1500, 40)])
def test_score(dt, d, B, H, Hkv, L, W):
    x = workloads.small_random(B, H, Hkv, L, d, seed=13, dtype=dt)
    s = host(tsa.score(dev(x["q"], dt), dev(x["k"], dt), W))
    want = oracle.score(x["q"], x["k"], W)
    err = rel_err(s, want)
    print(f"score {dt} L={L} W={W}: max rel err {err:.3e}")
    assert err <= 1e-5
    np.testing.assert_allclose(s.sum(-1), min(W, L), rtol=1e-5)


def test_score_zero_query_exact_ties():
    # q = 0: every key before the window gets the same score H_L - H_{L-W}; the GPU sums
    # the same fp32 terms in the same order for every key, so they tie exactly.
    L, W = 3000, 64
    x = workloads.small_random(1, 4, 2, L, 128, seed=1, dtype="bf16")
    q = torch.zeros(1, L, 4, 128, dtype=torch.bfloat16, device="cuda")
    s = tsa.score(q, dev(x["k"], "bf16"), W).cpu().numpy()
    head = s[:, :, : L - W]
    assert np.all(head == head[:, :, :1])
    want = sum(1.0 / m for m in range(L - W + 1, L + 1))
    assert abs(float(head[0, 0, 0]) - want) <= 1e-6 * want
    idx = tsa.select(torch.from_numpy(s).cuda(), 500, W, 4).cpu().numpy()
    assert idx[0, 0].tolist() == list(range(500 - W)) + list(range(L - W, L))


# ---- end to end ---------------------------------------------------------------------------

def _end_to_end(x, dt, keep, W, ns, in_place=False, per_kv_head=False):
    q, k, v, r = (dev(x[n], dt) for n in "qkvr")
    Hkv = x["k"].shape[2]
    kvh = Hkv if per_kv_head else None
    if in_place:
        out = r.clone()
        _, sg, ig = tsa.forward(q, k, v, out, keep, W, ns, out=out, return_scores=True, per_kv_head=per_kv_head)
    else:
        out, sg, ig = tsa.forward(q, k, v, r, keep, W, ns, return_scores=True, per_kv_head=per_kv_head)
    s32 = sg.cpu().numpy()
    s_gpu = s32.astype(np.float64)
    idx = ig.cpu().numpy().astype(np.int64)
    s_or = oracle.score(x["q"], x["k"], W)
    print(f"score max rel err {rel_err(s_gpu, s_or):.3e}")
    assert rel_err(s_gpu, s_or) <= 1e-5
    # select stage bit-exact on its own input (per KV head: summed in fp32, as the kernel does)
    assert np.array_equal(idx, oracle.select(s32, keep, W, ns, kvh))
    n_diff = check_selection(oracle.group_scores(s_or, Hkv) if per_kv_head else s_or, idx, keep, W, ns)
    qh, kh, vh = oracle.gather(x["q"], x["k"], x["v"], idx)
    oh_or = oracle.attend(qh, kh, vh)
    # Attention stage on the GPU's own subset: the 1e-4 / 2e-2 bar.
    ig = torch.from_numpy(idx.astype(np.int32)).cuda()
    oh_gpu = host(tsa.attn(*tsa.gather_qkv(q, k, v, ig)))
    att_err = float(np.max(np.abs(oh_gpu - oh_or)))
    assert att_err <= TOL[dt]
    # Final output: unselected rows are the residual bit for bit; a selected row is the
    # residual plus attention rounded once more to the storage dtype, so it may differ
    # from the exact value by the attention bar plus half a spacing of that dtype.
    want = oracle.scatter_residual(oh_or, idx, x["r"])
    got = host(out)
    B, L, H, _ = x["q"].shape
    sel = np.zeros((B, L, H), dtype=bool)
    SG = H // idx.shape[1]
    for b in range(B):
        for h in range(H):
            sel[b, idx[b, h // SG], h] = True
    assert np.array_equal(got[~sel], x["r"][~sel].astype(np.float64))
    excess = np.abs(got[sel] - want[sel]) - half_ulp(got[sel], dt)
    err = float(np.max(np.abs(got[sel] - round_to(want[sel], dt))))
    print(f"end-to-end {dt}{' per KV head' if per_kv_head else ''}: attn err {att_err:.3e}, "
          f"out err vs once-rounded oracle {err:.3e}, "
          f"excess over half-ulp {excess.max():.3e}, subset differences {n_diff}")
    assert excess.max() <= TOL[dt]


def test_forward_fp32_L512_config():
    w = workloads.WORKLOADS["fp32_L512"]
    _end_to_end(workloads.make_inputs(w), "fp32", w.keep, w.W, w.n_sink)


@pytest.mark.parametrize("B,H,Hkv,L,d,keep,W,ns,in_place", [
    (2, 8, 2, 1234, 128, 500, 64, 4, False),
    (1, 8, 2, 1234, 128, 500, 64, 4, True),
    (1, 4, 4, 999, 64, 300, 32, 4, False),
    (1, 4, 1, 100, 128, 100, 64, 4, False),
])
def test_forward_bf16(B, H, Hkv, L, d, keep, W, ns, in_place):
    x = workloads.small_random(B, H, Hkv, L, d, seed=L + keep, dtype="bf16")
    _end_to_end(x, "bf16", keep, W, ns, in_place)


def test_forward_fp32_in_place():
    x = workloads.small_random(1, 4, 2, 640, 64, seed=4, dtype="fp32")
    _end_to_end(x, "fp32", 200, 32, 4, in_place=True)


@pytest.mark.parametrize("case", ["case1", "case2"])
def test_hand_cases_through_gpu(case):
    # The hand-worked cases, embedded in d = 64 (zero padding; scale 1/8, so the key
    # entry is 8 ln 2 for a logit of ln 2), fp32.
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))
    c, e = g["common"], g[case]
    L, d = c["L"], 64

    def num(s):
        from fractions import Fraction
        return float(Fraction(s)) if isinstance(s, str) else float(s)

    q = np.zeros((1, L, 1, d), np.float32)
    k = np.zeros((1, L, 1, d), np.float32)
    for p in e["q_nonzero"]:
        q[0, int(p), 0, 0] = 1.0
    for p in e["k_nonzero"]:
        k[0, int(p), 0, 0] = 8.0 * math.log(2.0)
    v = np.zeros((1, L, 1, d), np.float32)
    r = np.zeros((1, L, 1, d), np.float32)
    v[0, :, 0, :2] = np.array(c["v"], np.float32)
    r[0, :, 0, :2] = np.array(c["r"], np.float32)
    out, s, idx = tsa.forward(dev(q), dev(k), dev(v), dev(r), c["keep"], c["W"], c["n_sink"], return_scores=True)
    assert idx.cpu().numpy()[0, 0].tolist() == e["idx"]
    np.testing.assert_allclose(s.cpu().numpy()[0, 0], [num(t) for t in e["scores"]], rtol=1e-6)
    want = np.array([[num(t) for t in row] for row in e["out"]])
    np.testing.assert_allclose(host(out)[0, :, 0, :2], want, rtol=0, atol=1e-5)
    assert np.all(host(out)[0, :, 0, 2:] == 0)


@pytest.mark.parametrize("B,H,Hkv,L,d,keep,in_place", [(2, 8, 2, 1234, 128, 500, False), (1, 8, 2, 1234, 128, 500, True),
                                                      (1, 4, 4, 999, 64, 300, False), (1, 4, 1, 3000, 128, 3000, False)])
def test_fused_forward_equals_staged(B, H, Hkv, L, d, keep, in_place):
    # The bf16 forward reads rows through the index lists and writes residual + O from the
    # attention epilogue; it must equal the staged entry points (gather, attention on the
    # compact rows, scatter + residual) bit for bit.
    x = workloads.small_random(B, H, Hkv, L, d, seed=17, dtype="bf16")
    q, k, v, r = (dev(x[n], "bf16") for n in "qkvr")
    if in_place:
        out = r.clone()
        _, s_f, idx = tsa.forward(q, k, v, out, keep, 64, 4, out=out, return_scores=True)
    else:
        out, s_f, idx = tsa.forward(q, k, v, r, keep, 64, 4, return_scores=True)
    staged = tsa.scatter_residual(tsa.attn(*tsa.gather_qkv(q, k, v, idx)), idx, r)
    assert torch.equal(out, staged)
    assert torch.equal(tsa.score(q, k, 64), s_f)
    assert torch.equal(tsa.select(s_f, keep, 64, 4), idx)


@pytest.mark.parametrize("L,keep,W,ns", [
    (40, 40, 64, 4),        # window covers the sequence, one partial key tile
    (65, 36, 32, 4),        # keep = |F|: no score-chosen token; a ragged second tile
    (200, 200, 64, 4),      # keep = L: sparse must equal dense
    (129, 70, 1, 1),        # one-row window
    (8, 3, 1, 1),           # the tiny case
])
def test_fused_forward_edge_cases(L, keep, W, ns):
    x = workloads.small_random(1, 4, 2, L, 128, seed=L, dtype="bf16")
    q, k, v, r = (dev(x[n], "bf16") for n in "qkvr")
    out, s_f, idx = tsa.forward(q, k, v, r, keep, W, ns, return_scores=True)
    staged = tsa.scatter_residual(tsa.attn(*tsa.gather_qkv(q, k, v, idx)), idx, r)
    assert torch.equal(out, staged)
    _end_to_end(x, "bf16", keep, W, ns)
    if keep == L:
        dense = tsa.dense_attn(q, k, v).float() + r.float()
        assert float((out.float() - dense).abs().max()) <= 2e-2 + 0.0625


def test_deterministic():
    x = workloads.small_random(1, 8, 2, 2000, 128, seed=3, dtype="bf16")
    q, k, v, r = (dev(x[n], "bf16") for n in "qkvr")
    a = tsa.forward(q, k, v, r, 700, 64, 4, return_scores=True)
    b = tsa.forward(q, k, v, r, 700, 64, 4, return_scores=True)
    for ta, tb in zip(a, b):
        assert torch.equal(ta, tb)


# ---- token subsets shared per KV head ----------------------------------------------------

@pytest.mark.parametrize("B,H,Hkv,L,keep,W,ns,ties", [
    (1, 8, 2, 1000, 137, 5, 3, False),
    (2, 4, 1, 777, 300, 64, 4, True),
    (1, 6, 3, 513, 68, 64, 4, False),        # keep = |F|
    (1, 4, 4, 300, 100, 8, 2, True),         # one query head per KV head
    (1, 32, 8, 131072, 32768, 64, 4, True),
])
def test_select_per_kv_head_bitexact(B, H, Hkv, L, keep, W, ns, ties):
    rng = np.random.default_rng(L + H)
    s = rng.random((B, H, L)).astype(np.float32) * 0.01
    if ties:
        s = (np.round(s * 200) / 200).astype(np.float32)
    s[..., :ns] = 0.0
    idx = tsa.select(torch.from_numpy(s).cuda(), keep, W, ns, kv_heads=Hkv).cpu().numpy()
    assert idx.shape == (B, Hkv, keep)
    assert np.array_equal(idx, oracle.select(s, keep, W, ns, kv_heads=Hkv))


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("fp32", 64)])
def test_gather_scatter_per_kv_head_bitexact(dt, d):
    B, H, Hkv, L, keep = 2, 8, 2, 300, 77
    x = workloads.small_random(B, H, Hkv, L, d, seed=23, dtype=dt)
    rng = np.random.default_rng(6)
    idx = np.stack([np.stack([np.sort(rng.choice(L, keep, replace=False)) for _ in range(Hkv)]) for _ in range(B)])
    q, k, v, r = (dev(x[n], dt) for n in "qkvr")
    ig = torch.from_numpy(idx.astype(np.int32)).cuda()
    qh, kh, vh = tsa.gather_qkv(q, k, v, ig)
    assert tuple(kh.shape) == (B, Hkv, keep, d)
    wq, wk, wv = oracle.gather(x["q"], x["k"], x["v"], idx)
    assert np.array_equal(host(qh), wq) and np.array_equal(host(kh), wk) and np.array_equal(host(vh), wv)
    oh_vals = rng.standard_normal((B, H, keep, d)).astype(np.float32)
    oh_vals = workloads.round_bf16(oh_vals) if dt == "bf16" else oh_vals
    oh = dev(oh_vals, dt)
    want = round_to(oracle.scatter_residual(oh_vals, idx, x["r"]), dt)
    assert np.array_equal(host(tsa.scatter_residual(oh, ig, r)), want)
    r2 = r.clone()
    tsa.scatter_residual(oh, ig, r2, out=r2)
    assert np.array_equal(host(r2), want)


# bf16 with an even group size runs two query heads per workgroup on shared K/V tiles.
@pytest.mark.parametrize("dt,d,n,B,H,Hkv", [("bf16", 128, 300, 1, 8, 2), ("bf16", 128, 1000, 1, 8, 2),
                                           ("bf16", 128, 500, 2, 8, 4), ("bf16", 128, 400, 2, 6, 2),
                                           ("bf16", 64, 257, 1, 8, 2), ("fp32", 128, 200, 1, 8, 2)])
def test_attn_per_kv_head(dt, d, n, B, H, Hkv):
    rng = np.random.default_rng(n + d + 1)
    qh = rng.standard_normal((B, H, n, d)).astype(np.float32)
    kh, vh = (rng.standard_normal((B, Hkv, n, d)).astype(np.float32) for _ in range(2))
    if dt == "bf16":
        qh, kh, vh = (workloads.round_bf16(t) for t in (qh, kh, vh))
    oh = tsa.attn(dev(qh, dt), dev(kh, dt), dev(vh, dt))
    err = np.max(np.abs(host(oh) - oracle.attend(qh, kh, vh)))
    print(f"attn per KV head {dt} d={d} n={n}: max abs err {err:.3e}")
    assert err <= TOL[dt]


@pytest.mark.parametrize("B,H,Hkv,L,d,keep,W,ns,in_place", [
    (1, 8, 2, 1000, 128, 400, 64, 4, False),
    (2, 8, 4, 700, 128, 300, 16, 2, True),
    (1, 4, 1, 513, 64, 200, 64, 4, False),
    (1, 6, 2, 600, 128, 250, 32, 4, False),     # group of 3: one head per workgroup
])
def test_forward_bf16_per_kv_head(B, H, Hkv, L, d, keep, W, ns, in_place):
    x = workloads.small_random(B, H, Hkv, L, d, seed=31, dtype="bf16")
    _end_to_end(x, "bf16", keep, W, ns, in_place=in_place, per_kv_head=True)


def test_forward_fp32_per_kv_head():
    x = workloads.small_random(1, 4, 2, 512, 64, seed=32, dtype="fp32")
    _end_to_end(x, "fp32", 256, 32, 4, per_kv_head=True)
    _end_to_end(x, "fp32", 256, 32, 4, in_place=True, per_kv_head=True)


@pytest.mark.parametrize("in_place", [False, True])
def test_fused_equals_staged_per_kv_head(in_place):
    x = workloads.small_random(2, 8, 2, 1234, 128, seed=18, dtype="bf16")
    q, k, v, r = (dev(x[n], "bf16") for n in "qkvr")
    if in_place:
        out = r.clone()
        _, s_f, idx = tsa.forward(q, k, v, out, 500, 64, 4, out=out, return_scores=True, per_kv_head=True)
    else:
        out, s_f, idx = tsa.forward(q, k, v, r, 500, 64, 4, return_scores=True, per_kv_head=True)
    assert tuple(idx.shape) == (2, 2, 500)
    staged = tsa.scatter_residual(tsa.attn(*tsa.gather_qkv(q, k, v, idx)), idx, r)
    assert torch.equal(out, staged)
    assert torch.equal(tsa.select(s_f, 500, 64, 4, kv_heads=2), idx)
