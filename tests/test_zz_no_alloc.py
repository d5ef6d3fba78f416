"""tsa_forward_noalloc (the forward on the library's static per-GPU scratch array, no
workspace) against tsa_forward (caller's workspace) through the C ABI: scores, subsets and
output bit for bit, on consecutive calls that reuse the array, the second with a smaller
input, and across the forward's variants (per head, per KV head, adaptive budgets, fp32
staged, in place) up to the L = 131072 layer."""
import numpy as np
import pytest
import torch

import workloads
from tests._lib import ensure_built
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu

tsa = ensure_built()


def _pair(x, dt, keep, W=64, ns=4, per_kv=False, tau=0.0, in_place=False):
    q, k, v, r = (dev(x[n], dt) if isinstance(x[n], np.ndarray) else x[n] for n in "qkvr")
    desc = tsa.desc_for(q, k, keep, W, ns, per_kv_head=per_kv, tau=tau)
    B, L, H, _ = q.shape
    R = k.shape[2] if per_kv else H
    ws = torch.empty(tsa.tsa_workspace_size(desc, tsa.TSA_OP_FORWARD), dtype=torch.uint8, device="cuda")
    outs = []
    for noalloc in (False, True):
        out = r.clone() if in_place else torch.full_like(r, float("nan"))
        res = out if in_place else r
        scores = torch.full((B, H, L), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((B, R, desc.keep), -7, dtype=torch.int32, device="cuda")
        if noalloc:
            tsa.tsa_forward_noalloc(desc, q, k, v, res, out, scores, idx)
        else:
            tsa.tsa_forward(desc, q, k, v, res, out, scores, idx, ws)
        outs.append((out, scores, idx))
    torch.cuda.synchronize()
    (o1, s1, i1), (o2, s2, i2) = outs
    assert torch.equal(s1, s2)
    assert torch.equal(i1, i2)
    assert torch.equal(o1, o2)
    return o2


def test_noalloc_two_calls_second_smaller():
    # The array keeps the first call's contents; the second, smaller call must not depend on them.
    big = workloads.small_random(2, 8, 2, 3000, 128, seed=1, dtype="bf16")
    small = workloads.small_random(1, 8, 2, 1000, 128, seed=2, dtype="bf16")
    print("noalloc call 1: B=2 H=8 Hkv=2 L=3000 keep 1200", flush=True)
    _pair(big, "bf16", 1200)
    print("noalloc call 2: B=1 H=8 Hkv=2 L=1000 keep 400", flush=True)
    _pair(small, "bf16", 400)


@pytest.mark.parametrize("dt,B,H,Hkv,L,d,keep,per_kv,tau,in_place", [
    ("bf16", 1, 8, 2, 1234, 128, 500, True, 0.0, False),
    ("bf16", 1, 8, 2, 1500, 128, 1500, False, 0.3, False),
    ("bf16", 1, 4, 4, 999, 64, 300, False, 0.0, True),
    ("fp32", 1, 4, 4, 512, 64, 256, False, 0.0, False),
    ("fp32", 1, 4, 2, 640, 64, 200, False, 0.0, True),
])
def test_noalloc_variants(dt, B, H, Hkv, L, d, keep, per_kv, tau, in_place):
    print(f"noalloc {dt} B={B} H={H} Hkv={Hkv} L={L} d={d} keep={keep} per_kv={per_kv} tau={tau} "
          f"in_place={in_place}", flush=True)
    x = workloads.small_random(B, H, Hkv, L, d, seed=L, dtype=dt, q_grade=2.0)
    _pair(x, dt, keep, per_kv=per_kv, tau=tau, in_place=in_place)


def test_noalloc_full_size_layer():
    w = workloads.WORKLOADS["bf16_L128k_r0.5"]
    print("noalloc L=131072 keep 65536", flush=True)
    x = workloads.make_inputs(w)
    t = {n: torch.from_numpy(x[n]).to(torch.bfloat16).cuda() for n in "qkvr"}
    del x
    _pair(t, "bf16", w.keep)
