"""Helpers of the GPU parity tests: device transfer, exact rounding of oracle values to
the storage dtype, and the acceptance rules that compare the HIP path with the oracle."""
import numpy as np
import torch

import oracle

TOL = {"fp32": 1e-4, "bf16": 2e-2}
TORCH_DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


def dev(x, dt="fp32"):
    """Host float array holding dtype-exact values -> contiguous GPU tensor of that dtype."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(TORCH_DT[dt]).cuda()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def round_to(x, dt):
    """Round float64 values once to the storage dtype (nearest, ties to even)."""
    x = np.asarray(x, dtype=np.float64)
    if dt == "fp32":
        return x.astype(np.float32).astype(np.float64)
    m, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)   # 8 significant bits, np.rint ties to even


def half_ulp(x, dt):
    """Half the spacing of the storage dtype at each value of x (the rounding of one store)."""
    _, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(1.0, e - (9 if dt == "bf16" else 25))


def check_selection(s_or, idx_gpu, keep, W, n_sink, rel=1e-6):
    """End-to-end selection rule: per head, positions where the GPU subset differs from
    the oracle's must be non-forced and within rel * theta of the oracle threshold."""
    B, H, L = s_or.shape
    n_diff = 0
    for b in range(B):
        for h in range(H):
            S_or = set(oracle.select_row(s_or[b, h], keep, W, n_sink).tolist())
            S_gpu = idx_gpu[b, h].tolist()
            assert len(S_gpu) == keep and all(x < y for x, y in zip(S_gpu, S_gpu[1:]))
            F = set(oracle.forced_positions(L, W, n_sink).tolist())
            assert F <= set(S_gpu)
            diff = S_or.symmetric_difference(S_gpu)
            if diff:
                theta = oracle.threshold(s_or[b, h], keep, W, n_sink)
                for p in diff:
                    assert p not in F
                    assert abs(s_or[b, h, p] - theta) <= rel * theta, (b, h, p, s_or[b, h, p], theta)
                n_diff += len(diff)
    return n_diff


def check_adaptive_selection(s_or, idx_gpu, keep, W, n_sink, tau, rel=3e-5):
    """Token-coverage rule end to end, on float64 scores [B,H,L] and the GPU's padded subsets
    [B,H,keep]: per row, one more position leaving (the lowest-scoring non-forced member,
    ties to the higher position) would take the mass that left (every non-member) above tau
    of the row's total; below the cap (K < keep) the mass that left is within it (at the cap
    more leaves than coverage alone asks); both up to a relative slack `rel` (the GPU decides
    on its fp32 scores).  The members are the K best positions up to near-ties at the
    K-threshold (as in check_selection).  Returns the number of near-tie differences."""
    B, H, L = s_or.shape
    F = set(oracle.forced_positions(L, W, n_sink).tolist())
    tau32 = float(np.float32(tau))
    n_diff = 0
    for b in range(B):
        for h in range(H):
            row = np.asarray(s_or[b, h], dtype=np.float64)
            S = [int(p) for p in idx_gpu[b, h] if p >= 0]
            K = len(S)
            assert all(p < 0 for p in idx_gpu[b, h][K:]), "padding only after the members"
            assert all(x < y for x, y in zip(S, S[1:])) and F <= set(S)
            member = np.zeros(L, dtype=bool)
            member[S] = True
            budget = tau32 * row.sum()
            left = row[~member].sum()
            if K < keep:
                assert left <= budget * (1 + rel), (b, h, left, budget)
            movable = [p for p in S if p not in F]
            if movable:
                nxt = min(movable, key=lambda p: (row[p], -p))
                assert left + row[nxt] > budget * (1 - rel), (b, h, left, row[nxt], budget)
            S_or = set(oracle.select_row(row, K, W, n_sink).tolist())
            diff = S_or.symmetric_difference(S)
            if diff:
                theta = oracle.threshold(row, K, W, n_sink)
                for p in diff:
                    assert p not in F
                    assert abs(row[p] - theta) <= rel * theta, (b, h, p, row[p], theta)
                n_diff += len(diff)
    return n_diff


def rel_err(gpu, ref, floor=1e-30):
    return float(np.max(np.abs(gpu - ref) / np.maximum(np.abs(ref), floor)))
