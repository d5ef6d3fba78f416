"""The benchmark's roofline denominators and its one-GPU contract, checked on the CPU.

The work per stage that bench.py divides by a launch time is compared with figures
tabulated independently from the stage definitions and the workload shapes (rounded to
about four significant digits): flops of the score's window logits (one pass), of the
causal attention over the K kept rows and of dense causal attention over all L rows;
bytes of the score (K read once, the window queries, the scores written), of the select
(scores read, idx written), of the gather (Q, K, V rows read and written, idx read) and of
the out-of-place scatter (residual read, out written, O^ read).  The scatter here reads the
inverse map (4 B H L bytes) where the tabulated figure counts the index list (4 B H K)."""
import os
import subprocess
import sys

import pytest

import bench
import workloads

MB = 1e6
TABLE = {
    "bf16_L8k_r0.5": dict(score_flops=4.28e9, score_bytes=18.4 * MB, select_bytes=1.57 * MB,
                          gather_bytes=201.9 * MB, attn_flops=1.375e11, scatter_bytes=168.3 * MB,
                          dense_flops=5.498e11),
    "bf16_L32k_r0.25": dict(score_flops=1.72e10, score_bytes=71.8 * MB, select_bytes=5.24 * MB,
                            gather_bytes=403.7 * MB, attn_flops=5.498e11, scatter_bytes=605.0 * MB,
                            dense_flops=8.796e12),
    "bf16_L128k_r0.5": dict(score_flops=6.87e10, score_bytes=285.7 * MB, select_bytes=25.2 * MB,
                            gather_bytes=3229.6 * MB, attn_flops=3.518e13, scatter_bytes=2692.7 * MB,
                            dense_flops=1.407e14),
    "bf16_L128k_r0.25": dict(select_bytes=21.0 * MB, gather_bytes=1614.8 * MB, attn_flops=8.796e12,
                             scatter_bytes=2420.1 * MB),
    "bf16_L128k_r0.1": dict(select_bytes=18.5 * MB, gather_bytes=645.9 * MB, attn_flops=1.407e12,
                            scatter_bytes=2256.5 * MB),
    "bf16_L64k_planted": dict(score_flops=6.87e10, score_bytes=286.3 * MB, select_bytes=18.5 * MB,
                              gather_bytes=645.9 * MB, attn_flops=7.037e11, scatter_bytes=2256.5 * MB,
                              dense_flops=7.037e13),
}


@pytest.mark.parametrize("name", sorted(TABLE))
def test_algorithmic_work_matches_the_tabulated_sizes(name):
    w = workloads.WORKLOADS[name]
    got = bench.algorithmic(w)
    for key, want in TABLE[name].items():
        if key == "scatter_bytes":
            want = want - 4 * w.B * w.H * w.keep + 4 * w.B * w.H * w.L
        assert got[key] == pytest.approx(want, rel=3e-3), (key, got[key], want)


def test_score_work_counts_one_pass():
    # 2 d flops per window logit, each window row seeing the keys up to its own position.
    w = workloads.WORKLOADS["bf16_L128k_r0.5"]
    logits = sum(w.L - w.W + r + 1 for r in range(w.W))
    assert bench.algorithmic(w)["score_flops"] == 2.0 * w.B * w.H * w.d * logits


def test_more_than_one_gpu_is_refused():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode != 0
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""
