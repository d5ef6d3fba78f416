"""The acceptance rules the GPU tests apply to selections, checked on the CPU: they accept
the oracle's own selections and reject plausible mistakes (a dropped member, a wrong
budget, a missing forced position)."""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import check_adaptive_selection, check_selection


def _scores(B, H, L, seed):
    rng = np.random.default_rng(seed)
    s = rng.random((B, H, L)) ** 4          # a heavy low tail, like softmax column sums
    return s / s.sum(-1, keepdims=True) * 64.0


@pytest.mark.parametrize("tau", [0.05, 0.2, 0.5])
def test_adaptive_rule_accepts_the_oracle(tau):
    s = _scores(1, 3, 400, 1)
    idx = oracle.select(s, 300, 16, 4, tau=tau)
    assert check_adaptive_selection(s, idx, 300, 16, 4, tau) == 0


def test_adaptive_rule_accepts_the_cap():
    s = _scores(1, 2, 300, 2)
    idx = oracle.select(s, 100, 8, 2, tau=0.01)         # coverage would keep more than keep
    assert ((idx >= 0).sum(-1) == 100).all()
    assert check_adaptive_selection(s, idx, 100, 8, 2, 0.01) == 0


def test_adaptive_rule_rejects_one_extra_drop():
    s = _scores(1, 1, 400, 3)
    idx = oracle.select(s, 400, 16, 4, tau=0.2)
    row = [int(p) for p in idx[0, 0] if p >= 0]
    F = set(oracle.forced_positions(400, 16, 4).tolist())
    movable = [p for p in row if p not in F]
    drop = min(movable, key=lambda p: (s[0, 0, p], -p))
    bad = np.full_like(idx, -1)
    kept = [p for p in row if p != drop]
    bad[0, 0, :len(kept)] = kept
    with pytest.raises(AssertionError):
        check_adaptive_selection(s, bad, 400, 16, 4, 0.2)


def test_adaptive_rule_rejects_one_missing_drop():
    s = _scores(1, 1, 400, 4)
    idx = oracle.select(s, 400, 16, 4, tau=0.2)
    row = [int(p) for p in idx[0, 0] if p >= 0]
    outside = sorted(set(range(400)) - set(row), key=lambda p: (-s[0, 0, p], p))
    bad = np.full_like(idx, -1)
    kept = sorted(row + [outside[0]])              # the best position that left comes back
    bad[0, 0, :len(kept)] = kept
    with pytest.raises(AssertionError):
        check_adaptive_selection(s, bad, 400, 16, 4, 0.2)


def test_adaptive_rule_rejects_a_swapped_member():
    s = _scores(1, 1, 400, 5)
    idx = oracle.select(s, 400, 16, 4, tau=0.2)
    row = [int(p) for p in idx[0, 0] if p >= 0]
    F = set(oracle.forced_positions(400, 16, 4).tolist())
    best_member = max((p for p in row if p not in F), key=lambda p: s[0, 0, p])
    outside = sorted(set(range(400)) - set(row), key=lambda p: s[0, 0, p])
    kept = sorted([p for p in row if p != best_member] + [outside[0]])   # same K, wrong member
    bad = np.full_like(idx, -1)
    bad[0, 0, :len(kept)] = kept
    with pytest.raises(AssertionError):
        check_adaptive_selection(s, bad, 400, 16, 4, 0.2)


def test_fixed_rule_accepts_the_oracle_and_rejects_a_missing_forced_position():
    s = _scores(2, 2, 300, 6)
    idx = oracle.select(s, 120, 16, 4)
    assert check_selection(s, idx, 120, 16, 4) == 0
    bad = idx.copy()
    # replace sink position 0 by the best position outside the subset
    outside = sorted(set(range(300)) - set(idx[0, 0].tolist()), key=lambda p: -s[0, 0, p])
    bad[0, 0] = np.sort(np.concatenate([idx[0, 0][idx[0, 0] != 0], [outside[0]]]))
    with pytest.raises(AssertionError):
        check_selection(s, bad, 120, 16, 4)


def test_adaptive_rule_rejects_a_cap_that_coverage_does_not_need():
    # K = keep although coverage alone lets more positions leave: one more could leave.
    s = _scores(1, 1, 300, 7)
    idx = oracle.select(s, 300, 8, 2, tau=0.3)
    K = int((idx >= 0).sum())
    assert K < 300
    fixed = oracle.select(s, K + 20, 8, 2)        # the K + 20 best, as if capped at K + 20
    with pytest.raises(AssertionError):
        check_adaptive_selection(s, fixed, K + 20, 8, 2, 0.3)
