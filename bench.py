"""Benchmark of one token-sparse attention layer (score -> select -> gather -> attention ->
scatter + residual) on one MI355X, on seeded synthetic inputs resident in HBM.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-sweep]
                  [--no-cpu-baseline] [--no-dense]

A step is one tsa_forward call (all five stages, out-of-place scatter) on the workload.
Prints ONE JSON line: the headline is prefill tokens/s = B * L / step time at
L = 131072 (bf16, 32 query / 8 KV heads, d = 128, W = 64, 4 sinks, keep ratio 0.5), with
the per-stage times, the speedup over the library's own dense causal attention at the
same L, the keep-ratio sweep (0.5 / 0.25 / 0.1), the roofline of the attention kernel
(the dominant one) and the float64 oracle timed on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="bf16_L128k_r0.5")
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--no-configs", action="store_true", help="skip the other workloads (C1-C3, C5)")
    p.add_argument("--stage-reps", type=int, default=5)
    p.add_argument("--stage", choices=["score", "select", "gather", "attn", "scatter", "dense", "forward", "drift",
                                       "copy"],
                   help="run only this stage (after one full forward to make its inputs) --stage-reps times; "
                        "for profiler runs")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timer:
    """HIP events on torch's current stream, which is the stream every library call uses."""

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


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_bf16_L128k_r0.5_hbm_traffic.txt")
ATTN_SOURCES = ["token_sparse_attention_head_amd/csrc/attn.hip", "token_sparse_attention_head_amd/csrc/common.h"]


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, or None when it was taken on another workload or another attention source."""
    import hashlib
    if workload != "bf16_L128k_r0.5" or not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    for line in open(TRAFFIC_PROFILE):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.split()[0] if v.split() else ""
    h = hashlib.sha256()
    for p in ATTN_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    if fields.get("source_sha256") != h.hexdigest() or "hbm_bytes_per_launch" not in fields:
        return None
    return float(fields["hbm_bytes_per_launch"])


def algorithmic(w, per_kv_head=False):
    """Work the method must do per stage (flops or bytes), as defined for the roofline.
    With subsets per KV head the K/V rows are gathered once per subset (R = Hkv)."""
    e = 2 if w.dtype == "bf16" else 4
    B, H, Hkv, L, d, K, W = w.B, w.H, w.Hkv, w.L, w.d, w.keep, min(w.W, w.L)
    R = Hkv if per_kv_head else H
    score_flops = 2.0 * B * H * d * sum(L - W + r + 1 for r in range(W)) * 2   # two passes over the window logits
    return {
        "score_flops": score_flops,
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


def gpu_case(tsa, torch, timer, w, x, args, reps, steps, warmup, with_dense, per_kv_head=False):
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
    t0 = time.perf_counter()
    ms_events = timer.run(step, steps)
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    step_stats = stats(timer.each(step, steps))      # the same steps timed one by one
    graph_ms = graph_step_ms(torch, timer, step, steps)

    # Stage by stage through the standalone entry points, same sizes and buffers.
    scores = torch.empty(B, H, L, dtype=torch.float32, device="cuda")
    idx = torch.empty(B, R, w.keep, dtype=torch.int32, device="cuda")
    sws = torch.empty(max(1, tsa.tsa_workspace_size(desc, tsa.TSA_OP_SCORE)), dtype=torch.uint8, device="cuda")
    lws = torch.empty(max(1, tsa.tsa_workspace_size(desc, tsa.TSA_OP_SELECT)), dtype=torch.uint8, device="cuda")
    comp = [torch.empty(B, n, w.keep, D, dtype=dt, device="cuda") for n in (H, R, R, H)]
    cws = torch.empty(max(1, tsa.tsa_workspace_size(desc, tsa.TSA_OP_SCATTER)), dtype=torch.uint8, device="cuda")
    stages = {
        "score": lambda: tsa.tsa_score(desc, q, k, scores, sws),
        "select": lambda: tsa.tsa_select(desc, scores, idx, lws, lws.numel()),
        "gather": lambda: tsa.tsa_gather_qkv(desc, q, k, v, idx, comp[0], comp[1], comp[2]),
        "attn": lambda: tsa.tsa_attn(desc, comp[0], comp[1], comp[2], comp[3]),
        "scatter": lambda: tsa.tsa_scatter_residual(desc, comp[3], idx, r, out, cws),
    }
    stage_ms = {}
    for name, fn in stages.items():
        fn()
        stage_ms[name] = timer.run(fn, reps)
    # Each stage timed call by call (median, min), and the HBM-bound stages also cold: a
    # 1 GiB buffer is written before every call so the 256 MB Infinity Cache holds none of
    # the stage's inputs.
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    flush = lambda: scratch.fill_(1)   # noqa: E731
    stage_stats = {name: {"warm": stats(timer.each(fn, max(reps, 5)))} for name, fn in stages.items()}
    for name in ("gather", "scatter"):
        stage_stats[name]["cold"] = stats(timer.each(stages[name], max(reps, 5), flush))
    # Representation drift across the layer (residual in, out): a bandwidth-bound reduction.
    dws = torch.empty(max(1, tsa.tsa_workspace_size(desc, tsa.TSA_OP_DRIFT)), dtype=torch.uint8, device="cuda")
    dval = torch.empty((), dtype=torch.float64, device="cuda")
    drift = lambda: tsa.tsa_drift(desc, r, out, dval, dws)   # noqa: E731
    drift()
    stage_ms["drift"] = timer.run(drift, reps)
    stage_stats["drift"] = {"warm": stats(timer.each(drift, max(reps, 5))),
                            "cold": stats(timer.each(drift, max(reps, 5), flush))}
    del scratch
    # In-place scatter variant (out == residual touches only kept rows); on a copy.
    r2 = r.clone()
    stage_ms["scatter_inplace"] = timer.run(lambda: tsa.tsa_scatter_residual(desc, comp[3], idx, r2, r2), reps)
    del r2

    res = {"workload": w.name, "subsets": "per_kv_head" if per_kv_head else "per_head", "keep": w.keep,
           "ratio": round(w.keep / w.L, 4), "ms_per_step": ms_events,
           "wall_ms_per_step": wall_ms, "step_stats_ms": step_stats,
           "graph_ms_per_step": graph_ms, "graph_tokens_per_s": B * L / (graph_ms / 1e3),
           "tokens_per_s": B * L / (ms_events / 1e3), "stage_ms": stage_ms,
           "stage_stats_ms": stage_stats}
    a = algorithmic(w, per_kv_head)
    res["stage_rate"] = {
        "score_tflops": a["score_flops"] / (stage_ms["score"] * 1e-3) / 1e12,
        "select_gbs": a["select_bytes"] / (stage_ms["select"] * 1e-3) / 1e9,
        "gather_gbs": a["gather_bytes"] / (stage_ms["gather"] * 1e-3) / 1e9,
        "attn_tflops": a["attn_flops"] / (stage_ms["attn"] * 1e-3) / 1e12,
        "scatter_gbs": a["scatter_bytes"] / (stage_ms["scatter"] * 1e-3) / 1e9,
        "drift_gbs": a["drift_bytes"] / (stage_ms["drift"] * 1e-3) / 1e9,
    }
    peak_mm = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    res["stage_roofline"] = {
        name: {"bound": bound, "achieved": res["stage_rate"][key], "peak": peak,
               "unit": "TFLOP/s" if bound == "mfma" else "GB/s", "frac": res["stage_rate"][key] / peak}
        for name, key, bound, peak in (("score", "score_tflops", "mfma", peak_mm),
                                       ("select", "select_gbs", "hbm", PEAK_HBM_GBS),
                                       ("gather", "gather_gbs", "hbm", PEAK_HBM_GBS),
                                       ("attn", "attn_tflops", "mfma", peak_mm),
                                       ("scatter", "scatter_gbs", "hbm", PEAK_HBM_GBS),
                                       ("drift", "drift_gbs", "hbm", PEAK_HBM_GBS))}
    res["stage_rate_cold"] = {
        f"{n}_gbs": a[f"{n}_bytes"] / (stage_stats[n]["cold"]["median"] * 1e-3) / 1e9
        for n in ("gather", "scatter", "drift")}
    if with_dense:
        o = torch.empty_like(q)
        dense = lambda: tsa.tsa_dense_attn(desc, q, k, v, o)   # noqa: E731
        dense()
        dms = timer.run(dense, max(2, reps // 2))
        res["dense_ms"] = dms
        res["dense_tflops"] = a["dense_flops"] / (dms * 1e-3) / 1e12
        res["speedup_vs_dense"] = dms / ms_events
        res["graph_speedup_vs_dense"] = dms / graph_ms
        res["attn_speedup_vs_dense"] = dms / stage_ms["attn"]
        del o
    del ws, comp, out
    return res


def adaptive_case(tsa, torch, timer, w, steps, reps, dense_ms):
    """The layer under adaptive budgets (token coverage w.tau, cap w.keep) on a graded
    workload: step time, the spread of the row budgets, the attention work they imply
    (sum over heads of 2*d*K_h*(K_h+1)), and a fixed-budget step with the same total
    attention work spread evenly (keep = sqrt(mean K_h*(K_h+1))), which shows what the
    uneven rows cost."""
    import math
    import workloads
    log(f"generating inputs for {w.name}")
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
    budget_ms = timer.run(lambda: tsa.tsa_budget(desc, scores, counts, lws, lws.numel()), reps)
    select_ms = timer.run(lambda: tsa.tsa_select(desc, scores, idx, lws, lws.numel()), reps)
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
    """One forward to build the stage inputs, then only `name`, reps times.  `copy` is a
    plain 1 GiB device-to-device copy (torch), the reference for HBM byte counters."""
    if name == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        ms = timer.run(lambda: dst.copy_(src), reps)
        return {"stage": "copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30, "reps": reps, "avg_ms": ms}
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v, r = (torch.from_numpy(x[n]).to(dt).cuda() for n in "qkvr")
    desc = tsa.desc_for(q, k, w.keep, w.W, w.n_sink)
    B, L, H, D = q.shape
    scores = torch.empty(B, H, L, dtype=torch.float32, device="cuda")
    idx = torch.empty(B, H, w.keep, dtype=torch.int32, device="cuda")
    out = torch.empty_like(r)
    ws = torch.empty(tsa.tsa_workspace_size(desc, tsa.TSA_OP_FORWARD), dtype=torch.uint8, device="cuda")
    sws = torch.empty(max(1, tsa.tsa_workspace_size(desc, tsa.TSA_OP_SCORE)), dtype=torch.uint8, device="cuda")
    cws = torch.empty(max(1, tsa.tsa_workspace_size(desc, tsa.TSA_OP_SCATTER)), dtype=torch.uint8, device="cuda")
    lws = torch.empty(tsa.tsa_workspace_size(desc, tsa.TSA_OP_SELECT), dtype=torch.uint8, device="cuda")
    tsa.tsa_forward(desc, q, k, v, r, out, scores, idx, ws)
    comp = [torch.empty(B, H, w.keep, D, dtype=dt, device="cuda") for _ in range(4)]
    tsa.tsa_gather_qkv(desc, q, k, v, idx, comp[0], comp[1], comp[2])
    o = torch.empty_like(q) if name == "dense" else None
    dws = torch.empty(max(1, tsa.tsa_workspace_size(desc, tsa.TSA_OP_DRIFT)), dtype=torch.uint8, device="cuda")
    dval = torch.empty((), dtype=torch.float64, device="cuda")
    fns = {
        "score": lambda: tsa.tsa_score(desc, q, k, scores, sws),
        "select": lambda: tsa.tsa_select(desc, scores, idx, lws, lws.numel()),
        "gather": lambda: tsa.tsa_gather_qkv(desc, q, k, v, idx, comp[0], comp[1], comp[2]),
        "attn": lambda: tsa.tsa_attn(desc, comp[0], comp[1], comp[2], comp[3]),
        "scatter": lambda: tsa.tsa_scatter_residual(desc, comp[3], idx, r, out, cws),
        "dense": lambda: tsa.tsa_dense_attn(desc, q, k, v, o),
        "forward": lambda: tsa.tsa_forward(desc, q, k, v, r, out, None, None, ws),
        "drift": lambda: tsa.tsa_drift(desc, r, out, dval, dws),
    }
    ms = timer.run(fns[name], reps)
    return {"workload": w.name, "stage": name, "reps": reps, "avg_ms": ms}


def cpu_baseline(w, x, budget_s=20.0):
    """Time the float64 oracle on a bounded sample of the workload: one (batch, head)'s
    scores, subset, gather and scatter in full, and compact attention rows sampled evenly
    across the subset; the attention time is scaled by the causal row costs (row t costs
    t + 1 key visits), the head time by the number of heads."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    b, h, G = 0, 0, w.G
    t0 = time.perf_counter()
    qb = x["q"][b, :, h, :].astype(np.float64)
    kb = x["k"][b, :, h // G, :].astype(np.float64)
    s = oracle.score_head(qb, kb, w.W, 1.0 / np.sqrt(w.d))
    t_score = time.perf_counter() - t0
    S = oracle.select_row(s, w.keep, w.W, w.n_sink)
    t_select = time.perf_counter() - t0 - t_score
    qh, kh, vh = qb[S], kb[S], x["v"][b, S, h // G, :].astype(np.float64)
    t_head = time.perf_counter() - t0
    t_gather = t_head - t_score - t_select
    # Attention rows: grow the sample until it costs about half the budget.
    n = w.keep
    rows_total = n * (n + 1) / 2.0
    nr, t_att, cost = 16, 0.0, 0.0
    while True:
        rows = np.unique(np.linspace(0, n - 1, nr).astype(np.int64))
        t1 = time.perf_counter()
        oracle.attend_rows(qh, kh, vh, rows, 1.0 / np.sqrt(w.d))
        t_att = time.perf_counter() - t1
        cost = float(np.sum(rows + 1))
        if t_att > budget_s / 4 or nr >= n:
            break
        nr *= 2
    t2 = time.perf_counter()
    oracle.scatter_residual(np.zeros((1, 1, n, w.d)), S[None, None], x["r"][b:b + 1, :, h:h + 1, :])
    t_scatter = time.perf_counter() - t2
    per_head = t_head + t_scatter + t_att * rows_total / cost
    total = per_head * w.B * w.H
    heads = w.B * w.H
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = sorted({f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()})
    except Exception:  # pragma: no cover
        blas = []
    return {"value": w.B * w.L / total, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{w.name}: head (b=0,h=0) score+select+gather+scatter in full, {len(rows)} of {n} compact "
                      f"attention rows evenly spaced, scaled by causal row cost and by {heads} heads; "
                      f"{t_head + t_att + t_scatter:.1f} s of CPU work",
            "seconds_per_step_extrapolated": total,
            "seconds_per_stage_extrapolated": {"score": t_score * heads, "select": t_select * heads,
                                               "gather": t_gather * heads,
                                               "attention": t_att * rows_total / cost * heads,
                                               "scatter": t_scatter * heads},
            "host": {"cpu_model": cpu_model, "affinity_cores": len(os.sched_getaffinity(0)),
                     "numpy": np.__version__, "blas": blas}}


def copy_bandwidth(torch, timer, reps=10):
    """Measured HBM copy rate beside the published 8 TB/s: torch's device copy of a 1 GiB
    tensor (1 GiB read + 1 GiB written per call, far beyond the 256 MB Infinity Cache)."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ms = timer.run(lambda: dst.copy_(src), reps)
    del src, dst
    gbs = 2 * n / (ms * 1e-3) / 1e9
    return {"kernel": "torch copy_ of a 1 GiB device tensor", "bytes_per_call": 2 * n, "avg_ms": ms,
            "gbs": gbs, "frac_of_peak": gbs / PEAK_HBM_GBS}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer shards by KV-head group with no "
              "exchange, so one GPU's share is the measured unit", file=sys.stderr)
        sys.exit(2)
    import torch

    import token_sparse_attention_head_amd as tsa
    import workloads

    if not os.path.exists(tsa.LIB_PATH):
        from token_sparse_attention_head_amd import build
        build.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    timer = Timer(torch)

    w = workloads.WORKLOADS[args.workload]
    log(f"generating inputs for {w.name}")
    t0 = time.perf_counter()
    x = workloads.make_inputs(w)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")

    if args.stage:
        print(json.dumps(stage_only(tsa, torch, timer, w, x, args.stage, args.stage_reps)), flush=True)
        return
    head = gpu_case(tsa, torch, timer, w, x, args, args.stage_reps, args.steps, args.warmup, not args.no_dense)
    log(f"{w.name}: {head['ms_per_step']:.3f} ms/step, stages {json.dumps(head['stage_ms'])}")
    sweep = [head]
    if not args.no_sweep and w.name.startswith("bf16_L128k"):
        for name in ("bf16_L128k_r0.5", "bf16_L128k_r0.25", "bf16_L128k_r0.1"):
            if name == w.name:
                continue
            wi = workloads.WORKLOADS[name]
            res = gpu_case(tsa, torch, timer, wi, x, args, args.stage_reps, max(3, args.steps // 2), 1, False)
            if "dense_ms" in head:
                res["dense_ms"] = head["dense_ms"]
                res["speedup_vs_dense"] = head["dense_ms"] / res["ms_per_step"]
                res["graph_speedup_vs_dense"] = head["dense_ms"] / res["graph_ms_per_step"]
                res["attn_speedup_vs_dense"] = head["dense_ms"] / res["stage_ms"]["attn"]
            log(f"{wi.name}: {res['ms_per_step']:.3f} ms/step, stages {json.dumps(res['stage_ms'])}")
            sweep.append(res)
        # The same keep ratios with one token subset per KV head (the library's extension).
        for name in ("bf16_L128k_r0.5", "bf16_L128k_r0.25", "bf16_L128k_r0.1"):
            wi = workloads.WORKLOADS[name]
            res = gpu_case(tsa, torch, timer, wi, x, args, args.stage_reps, max(3, args.steps // 2), 1, False,
                           per_kv_head=True)
            if "dense_ms" in head:
                res["dense_ms"] = head["dense_ms"]
                res["speedup_vs_dense"] = head["dense_ms"] / res["ms_per_step"]
                res["graph_speedup_vs_dense"] = head["dense_ms"] / res["graph_ms_per_step"]
                res["attn_speedup_vs_dense"] = head["dense_ms"] / res["stage_ms"]["attn"]
            log(f"{wi.name} per KV head: {res['ms_per_step']:.3f} ms/step, stages {json.dumps(res['stage_ms'])}")
            sweep.append(res)
        # Adaptive budgets (token coverage) on heads graded from diffuse to concentrated.
        wa = workloads.WORKLOADS["bf16_L128k_tau0.2_graded"]
        res = adaptive_case(tsa, torch, timer, wa, max(3, args.steps // 2), args.stage_reps, head.get("dense_ms"))
        log(f"{wa.name}: {res['ms_per_step']:.3f} ms/step, K/L {json.dumps(res['keep_ratio_per_head'])}, "
            f"fixed budget with the same work {json.dumps(res['fixed_budget_same_work'])}")
        sweep.append(res)

    # The other configurations of the workload set (parity cases; reported, not the headline).
    configs = []
    if not args.no_configs and not args.no_sweep:
        for name in ("fp32_L512", "bf16_L8k_r0.5", "bf16_L32k_r0.25", "bf16_L64k_planted"):
            wi = workloads.WORKLOADS[name]
            xi = workloads.make_inputs(wi)
            res = gpu_case(tsa, torch, timer, wi, xi, args, args.stage_reps, max(3, args.steps // 2), 1,
                           name == "bf16_L32k_r0.25" and not args.no_dense)
            del xi
            keys = ("workload", "keep", "ratio", "ms_per_step", "tokens_per_s", "graph_ms_per_step", "stage_ms",
                    "stage_roofline", "dense_ms", "speedup_vs_dense", "attn_speedup_vs_dense")
            entry = {k: res[k] for k in keys if k in res}
            entry["shape"] = {"B": wi.B, "L": wi.L, "H": wi.H, "Hkv": wi.Hkv, "d": wi.d, "W": wi.W,
                              "n_sink": wi.n_sink, "dtype": wi.dtype}
            log(f"{name}: {res['ms_per_step']:.3f} ms/step, stages {json.dumps(res['stage_ms'])}")
            configs.append(entry)

    a = algorithmic(w)
    attn_ms = head["stage_ms"]["attn"]
    achieved = a["attn_flops"] / (attn_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    roofline = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                "traffic": measured_traffic(w.name), "traffic_unit": "HBM bytes per launch",
                "kernel": "attn_bf16_kernel<128, 8, ATT_COMPACT, 1> (tsa_attn)" if w.dtype == "bf16" else "attn_kernel<float> (tsa_attn)",
                "avg_launch_ms": attn_ms,
                "algorithmic_per_launch": f"2*B*H*d*keep*(keep+1) = {a['attn_flops']:.4e} flop"}
    copy = copy_bandwidth(torch, timer)
    for st in head["stage_roofline"].values():
        if st["bound"] == "hbm":
            st["frac_of_copy"] = st["achieved"] / copy["gbs"]
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        cpu = cpu_baseline(w, x)

    line = {
        "metric": "token-sparse attention prefill tokens/s + speedup vs dense at L=128K, bf16",
        "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1), bf16-rounded)",
        "config": {"workload": w.name, "B": w.B, "L": w.L, "H": w.H, "Hkv": w.Hkv, "d": w.d, "keep": w.keep,
                   "W": w.W, "n_sink": w.n_sink, "parallelism": "single GPU"},
        "speedup_vs_dense": head.get("speedup_vs_dense"), "dense_ms": head.get("dense_ms"),
        "step_stats_ms": head["step_stats_ms"],
        "graph_ms_per_step": head["graph_ms_per_step"], "graph_tokens_per_s": head["graph_tokens_per_s"],
        "stage_ms": head["stage_ms"], "stage_stats_ms": head["stage_stats_ms"], "stage_rate": head["stage_rate"],
        "stage_rate_cold": head["stage_rate_cold"], "stage_roofline": head["stage_roofline"],
        "sweep": sweep, "configs": configs, "hbm_copy": copy,
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
