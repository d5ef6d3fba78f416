"""Benchmark of one token-sparse attention layer (score -> select -> gather -> attention ->
scatter + residual) on one MI355X, on seeded synthetic inputs resident in HBM.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-sweep]
                  [--no-configs] [--no-cpu-baseline] [--no-dense] [--detail PATH]

A step is one tsa_forward call (all five stages, out-of-place output) on the workload,
by default L = 131072 (bf16, 32 query / 8 KV heads, d = 128, W = 64, 4 sinks, keep ratio
0.5).  The last stdout line is the headline JSON (under 2 KB): prefill tokens/s = B * L /
step time, the speedup over the library's own dense causal attention at the same L, the
keep-ratio sweep (0.5 / 0.25 / 0.1) in brief, the roofline of the dominant kernel (the
fused attention of the step, timed alone) and the float64 oracle timed on a bounded
sample on the host cores.  Stage times, per-call statistics, the per-KV-head and
adaptive sweeps and the other workloads go to stderr as short lines and, in full, to the
JSON file given by --detail.
"""
from __future__ import annotations

import argparse
import math
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 matrix / vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "token-sparse attention prefill tokens/s + speedup vs dense at L=128K, bf16"

STAGES = ("score", "select", "gather", "attn", "scatter", "fused_attn", "sparse_attn", "drift", "scatter_inplace")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="bf16_L128k_r0.5")
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--no-configs", action="store_true", help="skip the other workloads (fp32 L=512, L=8192, "
                                                              "L=32768, planted L=65536)")
    p.add_argument("--detail", help="write every measurement as JSON to this file")
    p.add_argument("--stage-reps", type=int, default=5)
    p.add_argument("--stage", choices=list(STAGES) + ["dense", "forward", "copy"],
                   help="run only this stage (after one full forward to make its inputs) --stage-reps times; "
                        "for profiler runs")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timer:
    """HIP events on torch's current stream, the stream every library call is given."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, reps):
        """Mean ms of `reps` back-to-back calls (one pair of events around them all)."""
        t = self.torch
        s = t.cuda.current_stream()
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        a.record(s)
        for _ in range(reps):
            fn()
        b.record(s)
        t.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def span(self, fn, min_reps, span_ms, max_reps=1000):
        """Mean ms of back-to-back calls over about `span_ms` of GPU time (at least min_reps
        calls), after about a third of that span of untimed calls: short calls are then timed
        in steady state, not in the clock ramp after an idle GPU.  Returns (ms, calls)."""
        est = max(self.run(fn, 1), 1e-3)
        for _ in range(min(max_reps, math.ceil(span_ms / 3 / est))):
            fn()
        n = int(min(max_reps, max(min_reps, math.ceil(span_ms / est))))
        return self.run(fn, n), n

    def each(self, fn, reps, flush=None):
        """ms of every call timed alone (events around each call); `flush` runs untimed
        before each call (cold runs)."""
        t = self.torch
        s = t.cuda.current_stream()
        ev = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(reps)]
        t.cuda.synchronize()
        for a, b in ev:
            if flush is not None:
                flush()
            a.record(s)
            fn()
            b.record(s)
        t.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]


def stats(ms):
    ms = sorted(ms)
    n = len(ms)
    med = ms[n // 2] if n % 2 else 0.5 * (ms[n // 2 - 1] + ms[n // 2])
    return {"median": med, "min": ms[0], "max": ms[-1], "n": n}


# HBM bytes per launch of the fused attention kernel, from the committed rocprofv3
# FETCH_SIZE / WRITE_SIZE summary, valid while the kernel sources and the build script (its
# compiler flags) hash as recorded there.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_fused_bf16_L128k_r0.5_hbm_traffic.txt")
ATTN_SOURCES = ["token_sparse_attention_head_amd/csrc/attn.hip", "token_sparse_attention_head_amd/csrc/common.h",
                "token_sparse_attention_head_amd/build.py"]


def attn_source_sha():
    h = hashlib.sha256()
    for p in ATTN_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()


def measured_traffic(workload):
    if workload != "bf16_L128k_r0.5" or not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    for line in open(TRAFFIC_PROFILE):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.split()[0] if v.split() else ""
    if fields.get("source_sha256") != attn_source_sha() or "hbm_bytes_per_launch" not in fields:
        return None
    return float(fields["hbm_bytes_per_launch"])


def algorithmic(w, per_kv_head=False):
    """Work the method must do per stage (flops or bytes) for the roofline.  The score is
    one pass over the window logits (its second pass recomputes them: executed work, not
    algorithmic).  With subsets per KV head K/V rows are gathered once per subset."""
    e = 2 if w.dtype == "bf16" else 4
    B, H, Hkv, L, d, K, W = w.B, w.H, w.Hkv, w.L, w.d, w.keep, min(w.W, w.L)
    R = Hkv if per_kv_head else H
    return {
        "score_flops": 2.0 * B * H * d * sum(L - W + r + 1 for r in range(W)),
        "score_bytes": B * Hkv * L * d * e + B * H * W * d * e + 4 * B * H * L,
        # scores read; per KV head also the summed rows written and read back; idx written
        "select_bytes": 4 * B * H * L + (8 * B * R * L if R < H else 0) + 4 * B * R * K,
        "gather_bytes": 2 * (B * H + 2 * B * R) * K * d * e + 4 * B * H * K,
        "attn_flops": 2.0 * B * H * d * K * (K + 1),
        "scatter_bytes": 2 * B * L * H * d * e + B * H * K * d * e + 4 * B * H * L,
        "dense_flops": 2.0 * B * H * d * L * (L + 1),
        "drift_bytes": 2 * B * L * H * d * e,          # both hidden-state tensors read once
    }


def graph_step_ms(torch, timer, step, steps):
    """ms per step when the whole step is captured once in a HIP graph and replayed (the
    launches of its kernels then cost no host round trips)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    ms = timer.run(g.replay, steps)
    del g
    return ms


STEP_SPAN_MS = 300.0    # GPU time each sweep or config step measurement covers
STAGE_SPAN_MS = 40.0    # and each stage measurement


def gpu_case(tsa, torch, timer, w, x, reps, steps, warmup, with_dense, per_kv_head=False, full=True, span=False):
    """One workload: the step (tsa_forward) and, with `full`, every stage through its own
    entry point, the fused attention alone, drift, cold runs and the dense reference.
    span=False: exactly `warmup` untimed and `steps` timed steps (the headline); span=True:
    steps over STEP_SPAN_MS of GPU time after a third of that untimed (the sweep and the
    other workloads, whose steps are short)."""
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v, r = (torch.from_numpy(x[n]).to(dt).cuda() for n in "qkvr")
    desc = tsa.desc_for(q, k, w.keep, w.W, w.n_sink, per_kv_head=per_kv_head)
    R = w.Hkv if per_kv_head else w.H
    ws = torch.empty(tsa.tsa_workspace_size(desc, tsa.TSA_OP_FORWARD), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(r)
    B, L, H, D = q.shape

    def step():
        tsa.tsa_forward(desc, q, k, v, r, out, None, None, ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if span:
        t0 = time.perf_counter()
        ms_events, steps = timer.span(step, steps, STEP_SPAN_MS)
        wall_ms = None
    else:
        t0 = time.perf_counter()
        ms_events = timer.run(step, steps)
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    res = {"workload": w.name, "subsets": "per_kv_head" if per_kv_head else "per_head", "keep": w.keep,
           "ratio": round(w.keep / w.L, 4), "ms_per_step": ms_events, "steps": steps, "wall_ms_per_step": wall_ms,
           "tokens_per_s": B * L / (ms_events / 1e3)}
    res["step_stats_ms"] = stats(timer.each(step, steps))      # the same steps timed one by one
    res["graph_ms_per_step"] = graph_ms = graph_step_ms(torch, timer, step, steps)
    res["graph_tokens_per_s"] = B * L / (graph_ms / 1e3)

    # Stage by stage through the standalone entry points, same sizes and buffers.
    scores = torch.empty(B, H, L, dtype=torch.float32, device="cuda")
    idx = torch.empty(B, R, w.keep, dtype=torch.int32, device="cuda")
    tsa.tsa_forward(desc, q, k, v, r, out, scores, idx, ws)
    sws = torch.empty(max(1, tsa.tsa_workspace_size(desc, tsa.TSA_OP_SCORE)), dtype=torch.uint8, device="cuda")
    lws = torch.empty(max(1, tsa.tsa_workspace_size(desc, tsa.TSA_OP_SELECT)), dtype=torch.uint8, device="cuda")
    aws = torch.empty(max(1, tsa.tsa_workspace_size(desc, tsa.TSA_OP_SPARSE_ATTN)), dtype=torch.uint8, device="cuda")
    r2 = r.clone()   # in-place target of the fused attention alone (accumulates; only timed)
    stages = {
        "score": lambda: tsa.tsa_score(desc, q, k, scores, sws),
        "select": lambda: tsa.tsa_select(desc, scores, idx, lws),
        # the step's own attention kernel: in place it is one fused launch
        "fused_attn": lambda: tsa.tsa_sparse_attn(desc, q, k, v, idx, r2, r2, aws),
        # out of place: inverse map + the fused attention launch, whose first workgroups copy
        # the unkept rows while the others run the attention
        "sparse_attn": lambda: tsa.tsa_sparse_attn(desc, q, k, v, idx, r, out, aws),
    }
    comp = None
    if full:
        comp = [torch.empty(B, n, w.keep, D, dtype=dt, device="cuda") for n in (H, R, R, H)]
        cws = torch.empty(max(1, tsa.tsa_workspace_size(desc, tsa.TSA_OP_SCATTER)), dtype=torch.uint8, device="cuda")
        stages.update({
            "gather": lambda: tsa.tsa_gather_qkv(desc, q, k, v, idx, comp[0], comp[1], comp[2]),
            "attn": lambda: tsa.tsa_attn(desc, comp[0], comp[1], comp[2], comp[3]),
            "scatter": lambda: tsa.tsa_scatter_residual(desc, comp[3], idx, r, out, cws),
        })
    stage_ms = {}
    for name, fn in stages.items():
        fn()
        stage_ms[name] = timer.span(fn, reps, STAGE_SPAN_MS)[0]
    res["stage_ms"] = stage_ms
    a = algorithmic(w, per_kv_head)
    peak_mm = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    rate = {
        "score": ("mfma", a["score_flops"] / (stage_ms["score"] * 1e-3) / 1e12, peak_mm),
        # the score sits near the ridge: its bytes (K once, the window queries, the scores
        # written) against the HBM roof as well
        "score_hbm": ("hbm", a["score_bytes"] / (stage_ms["score"] * 1e-3) / 1e9, PEAK_HBM_GBS),
        "select": ("hbm", a["select_bytes"] / (stage_ms["select"] * 1e-3) / 1e9, PEAK_HBM_GBS),
        "fused_attn": ("mfma", a["attn_flops"] / (stage_ms["fused_attn"] * 1e-3) / 1e12, peak_mm),
    }
    # What out of place adds to the in-place launch: the inverse map and the part of the
    # unkept-row copy the attention does not hide (no bandwidth figure: the copy overlaps).
    stage_ms["copy_exposed"] = stage_ms["sparse_attn"] - stage_ms["fused_attn"]
    if full:
        rate.update({
            "gather": ("hbm", a["gather_bytes"] / (stage_ms["gather"] * 1e-3) / 1e9, PEAK_HBM_GBS),
            "attn": ("mfma", a["attn_flops"] / (stage_ms["attn"] * 1e-3) / 1e12, peak_mm),
            "scatter": ("hbm", a["scatter_bytes"] / (stage_ms["scatter"] * 1e-3) / 1e9, PEAK_HBM_GBS),
        })
        # Each stage timed call by call, and the HBM-bound stages also cold: a 1 GiB buffer
        # is written before every call so the 256 MB Infinity Cache holds none of its inputs.
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        flush = lambda: scratch.fill_(1)   # noqa: E731
        st = {name: {"warm": stats(timer.each(fn, max(reps, 5)))} for name, fn in stages.items()}
        for name in ("gather", "scatter"):
            st[name]["cold"] = stats(timer.each(stages[name], max(reps, 5), flush))
        # Representation drift across the layer (residual in, out): a bandwidth-bound reduction.
        dws = torch.empty(max(1, tsa.tsa_workspace_size(desc, tsa.TSA_OP_DRIFT)), dtype=torch.uint8, device="cuda")
        dval = torch.empty((), dtype=torch.float64, device="cuda")
        drift = lambda: tsa.tsa_drift(desc, r, out, dval, dws)   # noqa: E731
        drift()
        stage_ms["drift"] = timer.run(drift, reps)
        rate["drift"] = ("hbm", a["drift_bytes"] / (stage_ms["drift"] * 1e-3) / 1e9, PEAK_HBM_GBS)
        st["drift"] = {"warm": stats(timer.each(drift, max(reps, 5))),
                       "cold": stats(timer.each(drift, max(reps, 5), flush))}
        del scratch
        res["stage_stats_ms"] = st
        res["stage_rate_cold_gbs"] = {n: a[f"{n}_bytes"] / (st[n]["cold"]["median"] * 1e-3) / 1e9
                                      for n in ("gather", "scatter", "drift")}
        r3 = r.clone()
        stage_ms["scatter_inplace"] = timer.run(lambda: tsa.tsa_scatter_residual(desc, comp[3], idx, r3, r3), reps)
        del r3
    res["stage_roofline"] = {n: {"bound": b_, "achieved": ach, "peak": pk, "unit": "TFLOP/s" if b_ == "mfma" else "GB/s",
                                 "frac": ach / pk} for n, (b_, ach, pk) in rate.items()}
    if with_dense:
        o = torch.empty_like(q)
        dense = lambda: tsa.tsa_dense_attn(desc, q, k, v, o)   # noqa: E731
        dense()
        dms = timer.run(dense, max(2, reps // 2))
        res["dense_ms"] = dms
        res["dense_tflops"] = a["dense_flops"] / (dms * 1e-3) / 1e12
        res["attn_stage_speedup_vs_dense"] = dms / stage_ms["fused_attn"]   # the attention stage alone
        del o
    del ws, comp, out, r2
    return res


def with_dense_ratios(res, dense_ms):
    if dense_ms:
        res["dense_ms"] = dense_ms
        res["speedup_vs_dense"] = dense_ms / res["ms_per_step"]
        res["graph_speedup_vs_dense"] = dense_ms / res["graph_ms_per_step"]
        res["attn_speedup_vs_dense"] = dense_ms / res["stage_ms"]["fused_attn"]
    return res


def adaptive_case(tsa, torch, timer, w, steps, reps, dense_ms):
    """The layer under adaptive budgets (token coverage w.tau, cap w.keep) on a graded
    workload: step time, the spread of the row budgets, the attention work they imply
    (sum over heads of 2*d*K_h*(K_h+1)), and a fixed-budget step with the same total
    attention work spread evenly (keep = sqrt(mean K_h*(K_h+1))), which shows what the
    uneven rows cost."""
    import workloads
    x = workloads.make_inputs(w)
    q, k, v, r = (torch.from_numpy(x[n]).to(torch.bfloat16).cuda() for n in "qkvr")
    del x
    B, L, H, D = q.shape
    desc = tsa.desc_for(q, k, w.keep, w.W, w.n_sink, tau=w.tau)
    ws = torch.empty(tsa.tsa_workspace_size(desc, tsa.TSA_OP_FORWARD), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(r)
    scores = torch.empty(B, H, L, dtype=torch.float32, device="cuda")
    step = lambda: tsa.tsa_forward(desc, q, k, v, r, out, None, None, ws)   # noqa: E731
    step()
    ms = timer.run(step, steps)
    tsa.tsa_forward(desc, q, k, v, r, out, scores, None, ws)
    counts = torch.empty(B, H, dtype=torch.int32, device="cuda")
    lws = torch.empty(tsa.tsa_workspace_size(desc, tsa.TSA_OP_SELECT), dtype=torch.uint8, device="cuda")
    idx = torch.empty(B, H, w.keep, dtype=torch.int32, device="cuda")
    budget_ms = timer.run(lambda: tsa.tsa_budget(desc, scores, counts, lws), reps)
    select_ms = timer.run(lambda: tsa.tsa_select(desc, scores, idx, lws), reps)
    K = counts.cpu().numpy().astype(np.float64)
    flops = float(np.sum(2.0 * D * K * (K + 1)))
    k_eq = int(round(math.sqrt(float(np.mean(K * (K + 1))))))
    fdesc = tsa.desc_for(q, k, k_eq, w.W, w.n_sink)
    fws = torch.empty(tsa.tsa_workspace_size(fdesc, tsa.TSA_OP_FORWARD), dtype=torch.uint8, device="cuda")
    fstep = lambda: tsa.tsa_forward(fdesc, q, k, v, r, out, None, None, fws)   # noqa: E731
    fstep()
    fixed_ms = timer.run(fstep, steps)
    res = {"workload": w.name, "subsets": "per_head_adaptive", "tau": w.tau, "keep_cap": w.keep,
           "ms_per_step": ms, "tokens_per_s": B * L / (ms / 1e3),
           "keep_ratio_per_head": {"min": K.min() / L, "mean": K.mean() / L, "max": K.max() / L},
           "attn_flops": flops, "attn_tflops_over_step": flops / (ms * 1e-3) / 1e12,
           "stage_ms": {"budget": budget_ms, "select_adaptive": select_ms},
           "fixed_budget_same_work": {"keep": k_eq, "ms_per_step": fixed_ms}}
    if dense_ms:
        res["dense_ms"] = dense_ms
        res["speedup_vs_dense"] = dense_ms / ms
    del q, k, v, r, ws, fws, out, scores
    return res


def stage_only(tsa, torch, timer, w, x, name, reps):
    """One forward to build the stage inputs, then only `name`, reps times.  `copy` is the
    library's plain device copy of 1 GiB, the reference of the HBM byte counters."""
    if name == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        ms = timer.run(lambda: tsa.tsa_stream_copy(dst, src), reps)
        return {"stage": "copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30, "reps": reps, "avg_ms": ms}
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v, r = (torch.from_numpy(x[n]).to(dt).cuda() for n in "qkvr")
    desc = tsa.desc_for(q, k, w.keep, w.W, w.n_sink)
    B, L, H, D = q.shape
    scores = torch.empty(B, H, L, dtype=torch.float32, device="cuda")
    idx = torch.empty(B, H, w.keep, dtype=torch.int32, device="cuda")
    out = torch.empty_like(r)
    ws = torch.empty(tsa.tsa_workspace_size(desc, tsa.TSA_OP_FORWARD), dtype=torch.uint8, device="cuda")
    tsa.tsa_forward(desc, q, k, v, r, out, scores, idx, ws)
    def wsp(op):
        return torch.empty(max(1, tsa.tsa_workspace_size(desc, op)), dtype=torch.uint8, device="cuda")
    comp = [torch.empty(B, H, w.keep, D, dtype=dt, device="cuda") for _ in range(4)] if name in (
        "gather", "attn", "scatter", "scatter_inplace") else None
    if comp is not None:
        tsa.tsa_gather_qkv(desc, q, k, v, idx, comp[0], comp[1], comp[2])
    o = torch.empty_like(q) if name == "dense" else None
    r2 = r.clone()
    dval = torch.empty((), dtype=torch.float64, device="cuda")
    fns = {
        "score": lambda ws_=wsp(tsa.TSA_OP_SCORE): tsa.tsa_score(desc, q, k, scores, ws_),
        "select": lambda ws_=wsp(tsa.TSA_OP_SELECT): tsa.tsa_select(desc, scores, idx, ws_),
        "gather": lambda: tsa.tsa_gather_qkv(desc, q, k, v, idx, comp[0], comp[1], comp[2]),
        "attn": lambda: tsa.tsa_attn(desc, comp[0], comp[1], comp[2], comp[3]),
        "scatter": lambda ws_=wsp(tsa.TSA_OP_SCATTER): tsa.tsa_scatter_residual(desc, comp[3], idx, r, out, ws_),
        "scatter_inplace": lambda: tsa.tsa_scatter_residual(desc, comp[3], idx, r2, r2),
        "fused_attn": lambda ws_=wsp(tsa.TSA_OP_SPARSE_ATTN): tsa.tsa_sparse_attn(desc, q, k, v, idx, r2, r2, ws_),
        "sparse_attn": lambda ws_=wsp(tsa.TSA_OP_SPARSE_ATTN): tsa.tsa_sparse_attn(desc, q, k, v, idx, r, out, ws_),
        "dense": lambda: tsa.tsa_dense_attn(desc, q, k, v, o),
        "forward": lambda: tsa.tsa_forward(desc, q, k, v, r, out, None, None, ws),
        "drift": lambda ws_=wsp(tsa.TSA_OP_DRIFT): tsa.tsa_drift(desc, r, out, dval, ws_),
    }
    ms = timer.run(fns[name], reps)
    return {"workload": w.name, "stage": name, "reps": reps, "avg_ms": ms}


# ---- the oracle on the host cores (a baseline, not the target) --------------------------

_ORACLE_X = None   # the workload's inputs, shared with the forked workers copy-on-write


def _oracle_head(job):
    """Worker: one (batch, query head) of the oracle -- scores, subset, gather and scatter
    in full, compact attention on evenly spaced rows until about `att_budget` seconds --
    and its seconds per stage, the attention scaled to every row by causal row cost."""
    import oracle
    b, h, G, W, n_sink, keep, d, att_budget = job
    x = _ORACLE_X
    scale = 1.0 / np.sqrt(d)
    t0 = time.perf_counter()
    qb = x["q"][b, :, h, :].astype(np.float64)
    kb = x["k"][b, :, h // G, :].astype(np.float64)
    s = oracle.score_head(qb, kb, W, scale)
    t1 = time.perf_counter()
    S = oracle.select_row(s, keep, W, n_sink)
    t2 = time.perf_counter()
    qh, kh, vh = qb[S], kb[S], x["v"][b, S, h // G, :].astype(np.float64)
    t3 = time.perf_counter()
    rows_total = keep * (keep + 1) / 2.0
    nr = 16
    while True:
        rows = np.unique(np.linspace(0, keep - 1, min(nr, keep)).astype(np.int64))
        ta = time.perf_counter()
        oh = oracle.attend_rows(qh, kh, vh, rows, scale)
        t_att = time.perf_counter() - ta
        if t_att > att_budget / 3 or nr >= keep:
            break
        nr *= 2
    cost = float(np.sum(rows + 1))
    t4 = time.perf_counter()
    full = np.zeros((1, 1, keep, d))
    full[0, 0, rows] = oh
    oracle.scatter_residual(full, S[None, None], x["r"][b:b + 1, :, h:h + 1, :])
    t5 = time.perf_counter()
    return {"score": t1 - t0, "select": t2 - t1, "gather": t3 - t2, "attention": t_att * rows_total / cost,
            "scatter": t5 - t4, "rows": len(rows), "measured": (t3 - t0) + t_att + (t5 - t4)}


def cpu_baseline(w, x, budget_s=20.0):
    """The float64 oracle on the host cores: a pool of single-threaded workers (one BLAS
    thread each) over the (batch, head) pairs, every pair's scores, subset, gather and
    scatter in full and its compact attention on a sample of rows scaled by causal row
    cost.  value = B * L / (extrapolated CPU seconds / workers).  Run before the GPU is
    touched, so the forked workers hold no GPU handles."""
    global _ORACLE_X
    import multiprocessing as mp
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    workers = max(1, min(16, cores))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    per_worker = -(-len(heads) // workers)
    att_budget = budget_s / per_worker
    _ORACLE_X = x

    def init():
        try:
            from threadpoolctl import threadpool_limits
            threadpool_limits(1)
        except Exception:  # pragma: no cover
            pass

    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers, initializer=init) as pool:
        out = pool.map(_oracle_head, [(b, h, w.G, w.W, w.n_sink, w.keep, w.d, att_budget) for b, h in heads])
    wall = time.perf_counter() - t0
    _ORACLE_X = None
    per_stage = {k: sum(o[k] for o in out) for k in ("score", "select", "gather", "attention", "scatter")}
    cpu_s = sum(per_stage.values())
    step_s = cpu_s / workers
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    rows = out[0]["rows"]
    return {"value": w.B * w.L / step_s, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"{w.name}: all {len(heads)} heads in full except compact attention, {rows} of {w.keep} "
                      f"rows per head scaled by causal row cost; {wall:.0f} s on {workers} single-threaded workers",
            "detail": {"seconds_per_step_extrapolated": step_s, "cpu_seconds_extrapolated": cpu_s,
                       "cpu_seconds_per_stage": per_stage, "measured_wall_s": wall,
                       "host": {"cpu_model": cpu_model, "affinity_cores": cores, "numpy": np.__version__,
                                "blas": _blas_info()}}}


def _blas_info():
    """BLAS libraries numpy loaded (name, version, threads), as threadpoolctl reports them."""
    try:
        from threadpoolctl import threadpool_info
        return [{k: i.get(k) for k in ("internal_api", "version", "num_threads")} for i in threadpool_info()
                if i.get("user_api") == "blas"]
    except Exception:  # pragma: no cover
        return "unknown"


# ---- main -------------------------------------------------------------------------------

def brief(res):
    """One short stderr line per measured workload."""
    parts = [f"{res['workload']} {res.get('subsets', '')}: {res['ms_per_step']:.3f} ms/step",
             f"{res['tokens_per_s']:.3e} tok/s"]
    if "speedup_vs_dense" in res:
        parts.append(f"{res['speedup_vs_dense']:.1f}x dense")
    if "stage_ms" in res:
        parts.append("stages " + " ".join(f"{k} {v:.3f}" for k, v in res["stage_ms"].items()))
    if "stage_roofline" in res:
        parts.append("frac " + " ".join(f"{k} {v['frac']:.2f}" for k, v in res["stage_roofline"].items()))
    return ", ".join(parts)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer shards by KV-head group with no "
              "exchange, so one GPU's share is the measured unit", file=sys.stderr)
        sys.exit(2)
    import workloads

    w = workloads.WORKLOADS[args.workload]
    t0 = time.perf_counter()
    x = workloads.make_inputs(w)
    log(f"inputs for {w.name} ready in {time.perf_counter() - t0:.1f} s")
    cpu = None
    if not args.no_cpu_baseline and not args.stage:
        cpu = cpu_baseline(w, x)
        log(f"oracle on the host: {cpu['value']:.1f} tokens/s ({cpu['sample']})")

    import torch

    import token_sparse_attention_head_amd as tsa

    if not os.path.exists(tsa.LIB_PATH):
        from token_sparse_attention_head_amd import build
        build.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    timer = Timer(torch)

    if args.stage:
        print(json.dumps(stage_only(tsa, torch, timer, w, x, args.stage, args.stage_reps)), flush=True)
        return
    head = gpu_case(tsa, torch, timer, w, x, args.stage_reps, args.steps, args.warmup, not args.no_dense)
    dense_ms = head.get("dense_ms")
    with_dense_ratios(head, dense_ms)
    log(brief(head))
    sweep = [head]
    if not args.no_sweep and w.name.startswith("bf16_L128k"):
        sub_steps = max(5, args.steps // 2)
        for name in ("bf16_L128k_r0.5", "bf16_L128k_r0.25", "bf16_L128k_r0.1"):
            for per_kv in (False, True):
                if name == w.name and not per_kv:
                    continue
                wi = workloads.WORKLOADS[name]
                res = gpu_case(tsa, torch, timer, wi, x, args.stage_reps, sub_steps, 1, False, per_kv, full=False,
                               span=True)
                sweep.append(with_dense_ratios(res, dense_ms))
                log(brief(res))
        wa = workloads.WORKLOADS["bf16_L128k_tau0.2_graded"]
        res = adaptive_case(tsa, torch, timer, wa, sub_steps, args.stage_reps, dense_ms)
        log(f"{wa.name}: {res['ms_per_step']:.3f} ms/step, K/L {res['keep_ratio_per_head']}, "
            f"fixed budget with the same work {res['fixed_budget_same_work']}")
        sweep.append(res)

    configs = []
    if not args.no_configs and not args.no_sweep:
        for name in ("fp32_L512", "bf16_L8k_r0.5", "bf16_L32k_r0.25", "bf16_L64k_planted"):
            wi = workloads.WORKLOADS[name]
            xi = workloads.make_inputs(wi)
            res = gpu_case(tsa, torch, timer, wi, xi, args.stage_reps, max(5, args.steps // 2), 1,
                           name == "bf16_L32k_r0.25" and not args.no_dense, span=True)
            del xi
            res = with_dense_ratios(res, res.get("dense_ms"))
            res["shape"] = {"B": wi.B, "L": wi.L, "H": wi.H, "Hkv": wi.Hkv, "d": wi.d, "W": wi.W,
                            "n_sink": wi.n_sink, "dtype": wi.dtype}
            log(brief(res))
            configs.append(res)

    # Measured copy bandwidth beside the published peak: the library's streaming copy of
    # 1 GiB (1 GiB read + 1 GiB written per call, far beyond the 256 MB Infinity Cache).
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    tsa.tsa_stream_copy(dst, src)
    cms = timer.run(lambda: tsa.tsa_stream_copy(dst, src), 10)
    del src, dst
    copy = {"kernel": "stream_copy_kernel (tsa_stream_copy), 1 GiB", "avg_ms": cms, "gbs": 2 * n / (cms * 1e-3) / 1e9}
    copy["frac_of_peak"] = copy["gbs"] / PEAK_HBM_GBS
    log(f"plain copy: {copy['gbs']:.0f} GB/s ({copy['frac_of_peak']:.2f} of 8 TB/s)")

    a = algorithmic(w)
    fused_ms = head["stage_ms"]["fused_attn"]
    achieved = a["attn_flops"] / (fused_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(w.name),
                "kernel": "attn_bf16_kernel<128,8,ATT_FUSED,1> (the step's attention, timed alone in place)"
                if w.dtype == "bf16" else "attn_kernel<float,...> (staged)",
                "avg_launch_ms": round(fused_ms, 4), "flop_per_launch": a["attn_flops"]}
    brief_sweep = {}
    for res in sweep:
        if res.get("subsets") == "per_head":
            brief_sweep[f"keep_{res['ratio']:g}"] = {
                "ms": round(res["ms_per_step"], 4), "tokens_per_s": round(res["tokens_per_s"]),
                "speedup_vs_dense": round(res["speedup_vs_dense"], 2) if "speedup_vs_dense" in res else None,
                "attn_frac": round(res["stage_roofline"]["fused_attn"]["frac"], 4)}
    line = {
        "metric": METRIC, "value": round(head["tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1), bf16-rounded)",
        "config": {"workload": w.name, "B": w.B, "L": w.L, "H": w.H, "Hkv": w.Hkv, "d": w.d, "keep": w.keep,
                   "W": w.W, "n_sink": w.n_sink, "parallelism": "single GPU"},
        "speedup_vs_dense": round(head["speedup_vs_dense"], 3) if "speedup_vs_dense" in head else None,
        "dense_ms": round(dense_ms, 3) if dense_ms else None,
        "graph_ms_per_step": round(head["graph_ms_per_step"], 4),
        "stage_ms": {k: round(v, 4) for k, v in head["stage_ms"].items()},
        "sweep": brief_sweep, "hbm_copy_gbs": round(copy["gbs"], 1), "roofline": roofline,
        "cpu_baseline": {k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample")} if cpu else None,
    }
    if args.detail:
        detail = dict(line, sweep=sweep, configs=configs, hbm_copy=copy, cpu_baseline=cpu)
        os.makedirs(os.path.dirname(os.path.abspath(args.detail)), exist_ok=True)
        with open(args.detail, "w") as f:
            json.dump(detail, f, indent=1)
        log(f"detail written to {args.detail}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
