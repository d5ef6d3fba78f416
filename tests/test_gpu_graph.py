"""The layer captured in a HIP graph (torch.cuda.CUDAGraph on ROCm): every replay, with the
program's own eager work and synchronisations between replays, equals the eager call bit for
bit.  The library launches only kernels on the caller's stream (no allocation, memset or
synchronisation inside a call), so a whole tsa_forward can be captured and replayed."""
import numpy as np
import pytest
import torch

import workloads
from tests._lib import ensure_built
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu

tsa = ensure_built()


@pytest.mark.parametrize("tau,per_kv_head,in_place", [(0.0, False, False), (0.2, False, False), (0.0, True, True)])
def test_forward_graph_replays_equal_eager(tau, per_kv_head, in_place):
    B, H, Hkv, L, d, keep, W, ns = 1, 8, 2, 1500, 128, 700, 64, 4
    x = workloads.small_random(B, H, Hkv, L, d, seed=3, dtype="bf16", q_grade=3.0)
    q, k, v, r = (dev(x[n], "bf16") for n in "qkvr")
    desc = tsa.desc_for(q, k, keep, W, ns, per_kv_head=per_kv_head, tau=tau)
    ws = torch.empty(tsa.tsa_workspace_size(desc, tsa.TSA_OP_FORWARD), dtype=torch.uint8, device="cuda")
    R = Hkv if per_kv_head else H
    idx = torch.empty(B, R, keep, dtype=torch.int32, device="cuda")

    def run(out):
        tsa.tsa_forward(desc, q, k, v, out if in_place else r, out, None, idx, ws)

    ref = r.clone()
    run(ref)
    torch.cuda.synchronize()
    ref_idx = idx.clone()

    out = r.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm-up on a side stream before capture
        run(out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out)
    for i in range(4):
        out.copy_(r)                                # eager work between replays
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        assert torch.equal(idx, ref_idx), f"replay {i}"
        other = r.clone()                           # an eager call between replays
        run(other)
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int16), ref.view(torch.int16))
