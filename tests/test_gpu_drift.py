"""Parity of the representation-drift kernel (skill page, Step 4) with the oracle.

Bar: |drift_gpu - drift_oracle| <= 2e-5.  Per token the kernel sums at most 64 fp32
products per lane and 6 butterfly levels, so a dot product or squared norm is off by at
most about 70 * 2^-24 (4.2e-6) of its magnitude bound |a||b| (Cauchy-Schwarz); with the
two norms, the square roots and the division a cosine is within about 1e-5, and so is
their mean (accumulated in fp64)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._lib import ensure_built
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu

tsa = ensure_built()
BAR = 2e-5


@pytest.mark.parametrize("dt,B,L,D", [("bf16", 2, 1000, 4096), ("bf16", 1, 1, 64), ("fp32", 1, 333, 384),
                                      ("fp32", 3, 50, 128), ("bf16", 1, 4099, 1024)])
def test_drift_matches_oracle(dt, B, L, D):
    rng = np.random.default_rng(L + D)
    a = rng.standard_normal((B, L, D)).astype(np.float32)
    b = (a + 0.3 * rng.standard_normal((B, L, D))).astype(np.float32)
    b[:, ::7] *= -1.0                        # some tokens reversed
    if dt == "bf16":
        a, b = workloads.round_bf16(a), workloads.round_bf16(b)
    got = float(tsa.drift(dev(a, dt), dev(b, dt)))
    want = oracle.drift(a, b)
    print(f"{dt} {B}x{L}x{D}: drift {got:.8f} oracle {want:.8f}")
    assert abs(got - want) <= BAR


def test_drift_closed_forms_and_determinism():
    rng = np.random.default_rng(1)
    a = workloads.round_bf16(rng.standard_normal((1, 777, 512)).astype(np.float32))
    ta = dev(a, "bf16")
    assert abs(float(tsa.drift(ta, ta))) <= BAR
    assert abs(float(tsa.drift(ta, -ta)) - 2.0) <= BAR
    z = torch.zeros_like(ta)
    assert abs(float(tsa.drift(ta, z)) - 1.0) <= BAR          # zero vectors: cosine 0
    tb = dev(workloads.round_bf16(rng.standard_normal((1, 777, 512)).astype(np.float32)), "bf16")
    d1, d2 = tsa.drift(ta, tb), tsa.drift(ta, tb)
    assert d1.item() == d2.item()


def test_drift_of_a_layer_L128k():
    # The drift across the L = 131072, keep 0.5 layer (residual in, out = residual + scattered
    # attention) at full size; the oracle runs over chunks of tokens and the chunk means are
    # combined with their token counts.
    w = workloads.WORKLOADS["bf16_L128k_r0.5"]
    x = workloads.make_inputs(w)
    q, k, v, r = (torch.from_numpy(x[n]).to(torch.bfloat16).cuda() for n in "qkvr")
    out = tsa.forward(q, k, v, r, w.keep, w.W, w.n_sink)
    del q, k, v
    got = float(tsa.drift(r, out))
    B, L, H, d = x["r"].shape
    o = out.float().cpu().numpy().reshape(B * L, H * d)
    rr = x["r"].reshape(B * L, H * d)
    step, acc = 8192, 0.0
    for t0 in range(0, B * L, step):
        n = min(step, B * L - t0)
        acc += n * (1.0 - oracle.drift(rr[t0:t0 + n], o[t0:t0 + n]))
    want = 1.0 - acc / (B * L)
    print(f"{w.name}: drift(residual, out) {got:.8f} oracle {want:.8f}")
    assert abs(got - want) <= BAR
