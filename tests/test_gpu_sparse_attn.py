"""Compress, attend and decompress on given subsets (tsa_sparse_attn) and the plain device
copy (tsa_stream_copy), through the C ABI.

tsa_sparse_attn must give exactly what the three staged entry points give on the same
index lists (gather, attention on the compact rows, scatter + residual; bit for bit), in
place and out of place, per head and per KV head, with fixed and adaptive (-1 padded)
budgets, bf16 (one fused kernel) and fp32 (staged through its workspace); and exactly
what tsa_forward writes for the subsets it chose.  The copy must be bit-exact and touch
nothing past its length."""
import numpy as np
import pytest
import torch

import workloads
from tests._lib import ensure_built
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu

tsa = ensure_built()


@pytest.mark.parametrize("dt,B,H,Hkv,L,d,keep,per_kv,tau,in_place", [
    ("bf16", 2, 8, 2, 1234, 128, 500, False, 0.0, False),
    ("bf16", 1, 8, 2, 1234, 128, 500, False, 0.0, True),
    ("bf16", 1, 8, 2, 1234, 128, 500, True, 0.0, False),
    ("bf16", 1, 4, 4, 999, 64, 300, False, 0.0, False),
    ("bf16", 1, 8, 2, 1500, 128, 1500, False, 0.3, False),   # adaptive budgets: -1 padded rows
    ("bf16", 1, 8, 2, 1500, 128, 1500, True, 0.3, True),
    ("fp32", 1, 4, 2, 640, 64, 200, False, 0.0, False),
    ("fp32", 1, 4, 2, 640, 64, 200, False, 0.0, True),
    ("fp32", 1, 4, 2, 640, 128, 640, False, 0.3, False),
])
def test_sparse_attn_equals_stages_and_forward(dt, B, H, Hkv, L, d, keep, per_kv, tau, in_place):
    x = workloads.small_random(B, H, Hkv, L, d, seed=L + keep, dtype=dt, q_grade=3.0)
    q, k, v, r = (dev(x[n], dt) for n in "qkvr")
    out_f, _, idx = tsa.forward(q, k, v, r, keep, 64, 4, return_scores=True, per_kv_head=per_kv, tau=tau)
    staged = tsa.scatter_residual(tsa.attn(*tsa.gather_qkv(q, k, v, idx)), idx, r)
    if in_place:
        out = r.clone()
        tsa.sparse_attn(q, k, v, idx, out, out=out, tau=tau)
    else:
        out = tsa.sparse_attn(q, k, v, idx, r, tau=tau)
    torch.cuda.synchronize()
    n_kept = int((idx >= 0).sum())
    print(f"{dt} {'per KV head' if per_kv else 'per head'} tau {tau} {'in place' if in_place else 'out of place'}: "
          f"{n_kept} kept rows")
    assert torch.equal(out, staged)
    assert torch.equal(out, out_f)
    if tau > 0:
        assert n_kept < idx.numel()                   # some rows really are padded


def test_sparse_attn_repeated_calls_are_identical():
    # Out of place the library rebuilds its inverse map in the workspace each call; a
    # second call on a workspace holding the first call's map gives the same bytes.
    x = workloads.small_random(1, 8, 2, 2000, 128, seed=3, dtype="bf16")
    q, k, v, r = (dev(x[n], "bf16") for n in "qkvr")
    _, _, idx = tsa.forward(q, k, v, r, 700, 64, 4, return_scores=True)
    desc = tsa.desc_for(q, k, 700, W=1, n_sink=0)
    ws = torch.empty(tsa.tsa_workspace_size(desc, tsa.TSA_OP_SPARSE_ATTN), dtype=torch.uint8, device="cuda")
    a, b = torch.empty_like(r), torch.full_like(r, 7.0)
    tsa.tsa_sparse_attn(desc, q, k, v, idx, r, a, ws)
    tsa.tsa_sparse_attn(desc, q, k, v, idx, r, b, ws)
    assert torch.equal(a, b)


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (64 << 20) + 48])
def test_stream_copy_bitexact(nbytes):
    g = torch.Generator().manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes + 64,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    tsa.tsa_stream_copy(dst, src, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert int(dst[nbytes:].count_nonzero()) == 0      # nothing past the length
    print(f"stream copy of {nbytes} bytes: exact", flush=True)


def test_copy_of_unkept_rows_all_keep_ratios():
    # The fused forward copies the residual to every row no head keeps (LDS-compacted row
    # lists per 1024 rows) and attention writes the kept ones: check every row of out is
    # written, for keep = |F| (almost every row copied) up to keep = L (none), per head and
    # per KV head, with a ragged last row block.
    x = workloads.small_random(1, 8, 2, 1500, 128, seed=9, dtype="bf16")
    q, k, v, r = (dev(x[n], "bf16") for n in "qkvr")
    for keep in (68, 300, 1499, 1500):
        for per_kv in (False, True):
            out = torch.full_like(r, float("nan"))
            _, _, idx = tsa.forward(q, k, v, r, keep, 64, 4, out=out, return_scores=True, per_kv_head=per_kv)
            sel = torch.zeros(1, idx.shape[1], 1500, dtype=torch.bool, device="cuda")
            sel.scatter_(2, idx.long(), True)
            sel = sel.repeat_interleave(8 // idx.shape[1], dim=1).permute(0, 2, 1)
            assert not torch.isnan(out.float()).any(), (keep, per_kv)
            assert torch.equal(out[~sel].view(torch.int16), r[~sel].view(torch.int16)), (keep, per_kv)


@pytest.mark.parametrize("B,H,Hkv,L,d,keep,W,ns,per_kv", [
    (1, 32, 8, 4096, 128, 400, 64, 4, False),   # copy inside the attention launch (64 rows per step)
    (3, 4, 2, 70, 128, 20, 8, 2, False),        # steps crossing batch entries (16 positions per step)
    (2, 8, 2, 3000, 64, 900, 64, 4, True),      # d = 64: 128 rows per step, per KV head
    (1, 6, 2, 2000, 128, 700, 64, 4, False),    # 6 heads do not divide a step: separate copy kernel
    (2, 2, 1, 20, 128, 10, 4, 1, False),        # L below a step's positions: separate copy kernel
    (1, 16, 4, 1500, 128, 1500, 64, 4, False),  # every row kept: nothing to copy
])
def test_out_of_place_equals_in_place(B, H, Hkv, L, d, keep, W, ns, per_kv):
    # The out-of-place forward copies the rows no head keeps (inside the attention launch
    # where the shape allows, else as its own kernel) and the attention writes the kept
    # rows; the in-place forward leaves unkept rows untouched.  Both must give the same
    # bytes, and every unkept row must equal the residual.
    x = workloads.small_random(B, H, Hkv, L, d, seed=B * L + H, dtype="bf16")
    q, k, v, r = (dev(x[n], "bf16") for n in "qkvr")
    out = torch.full_like(r, float("nan"))
    _, _, idx = tsa.forward(q, k, v, r, keep, W, ns, out=out, return_scores=True, per_kv_head=per_kv)
    r_in = r.clone()
    tsa.forward(q, k, v, r_in, keep, W, ns, out=r_in, per_kv_head=per_kv)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), r_in.view(torch.int16))
    sel = torch.zeros(B, idx.shape[1], L, dtype=torch.bool, device="cuda")
    sel.scatter_(2, idx.long(), True)
    sel = sel.repeat_interleave(H // idx.shape[1], dim=1).permute(0, 2, 1)
    assert torch.equal(out[~sel].view(torch.int16), r[~sel].view(torch.int16))
    print(f"B {B} H {H} L {L} d {d} keep {keep}: {int((~sel).sum())} unkept rows copied", flush=True)


def _random_shapes(n, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 8]))
        H = Hkv * G
        if H > 64:
            continue
        d = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 4))
        L = int(rng.integers(70, 3000))
        W = int(rng.choice([1, 16, 64]))
        ns = int(rng.integers(0, 5))
        forced = min(ns, L) + min(W, L)
        keep = int(rng.integers(min(forced, L), L + 1))
        per_kv = bool(rng.integers(0, 2)) and G > 1
        out.append((B, H, Hkv, L, d, keep, W, ns, per_kv))
    return out


@pytest.mark.parametrize("B,H,Hkv,L,d,keep,W,ns,per_kv", _random_shapes(14))
def test_out_of_place_equals_in_place_random_shapes(B, H, Hkv, L, d, keep, W, ns, per_kv):
    # Seeded random shapes over both copy paths (heads dividing a step's rows or not, rows
    # crossing batch entries, every keep ratio): out of place equals in place bit for bit.
    x = workloads.small_random(B, H, Hkv, L, d, seed=B * L + H + d, dtype="bf16")
    q, k, v, r = (dev(x[n], "bf16") for n in "qkvr")
    out = torch.full_like(r, float("nan"))
    tsa.forward(q, k, v, r, keep, W, ns, out=out, per_kv_head=per_kv)
    r_in = r.clone()
    tsa.forward(q, k, v, r_in, keep, W, ns, out=r_in, per_kv_head=per_kv)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), r_in.view(torch.int16))
