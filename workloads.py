"""Seeded synthetic workloads for Token Sparse Attention (shapes, dtypes, input draws).

This module holds the workload definitions and the seeded input generators that both
the oracle (``oracle/``) and the HIP path are fed from.  It contains none of the
method's arithmetic: no scoring, no selection, no attention.  It only draws numbers
and rounds them to the storage dtype.

Recipe (device independent, reproducible on any host):

* For each tensor in the order Q ``[B,L,H,d]``, K ``[B,L,Hkv,d]``, V ``[B,L,Hkv,d]``,
  R (residual) ``[B,L,H,d]``, and each block of ``ROWS_PER_BLOCK`` positions of each
  batch entry, an independent PCG64 stream is seeded from
  ``SeedSequence(seed, spawn_key=(tensor_id, b, block))`` and draws float32 standard
  normals.  Blocks are independent, so they are drawn on a thread pool.
* bf16 workloads round each float32 draw once to bfloat16, round-to-nearest-even.
  The same bf16 values go to the GPU (as raw bf16 bits) and, widened exactly, to the
  oracle.
* The planted-importance workload (two batch entries, L=65536) then, for every
  (batch, KV head) pair, picks 1% of the positions (655 of them) uniformly without
  replacement from ``[n_sink, L - W)`` with ``SeedSequence(seed, spawn_key=(4, b, g))``,
  forms the unit direction u of the mean of the last 64 queries of the heads in that
  KV group, and replaces each picked key by ``4 * |k| * u`` (then rounds to bf16).
  Picked tokens are never in the forced set, so only the scores can select them.
* Graded workloads (``q_grade`` > 1) multiply the float32 queries of head h by
  ``1 + (q_grade - 1) * h / (H - 1)`` before rounding, so the heads range from diffuse
  to concentrated attention (sharper logits) and adaptive budgets differ per head.
  N(0,1) draws alone give nearly uniform token scores, unlike the concentrated attention
  of trained models that token coverage is meant for.

The long-context workloads stand in for the long-context benchmark suites the paper
evaluates on (the pages give sequence lengths, not data): N(0,1) activations with
Llama-3-8B attention shapes (32 query heads, 8 KV heads, head dim 128).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

ROWS_PER_BLOCK = 4096
PLANT_FRACTION = 0.01
PLANT_SCALE = 4.0
PLANT_QUERY_ROWS = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    L: int
    d: int
    keep: int
    W: int
    n_sink: int
    dtype: str  # "fp32" or "bf16"
    planted: bool = False
    seed: int = 0
    tau: float = 0.0      # token coverage of adaptive budgets (0: every subset keeps `keep`)
    q_grade: float = 1.0  # query scale of the last head (graded workloads)

    @property
    def G(self) -> int:
        return self.H // self.Hkv

    @property
    def ratio(self) -> float:
        return self.keep / self.L

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _keep(ratio: float, L: int) -> int:
    # Subset size from a keep ratio: floor(ratio * L).
    return int(np.floor(ratio * L + 1e-9))


WORKLOADS = {
    # Single small fp32 layer, 4 heads without grouping.
    "fp32_L512": Workload("fp32_L512", 1, 4, 4, 512, 64, 256, 32, 4, "fp32"),
    # Llama-3-8B-shaped prefill layer (32 query heads / 8 KV heads, d=128).
    "bf16_L8k_r0.5": Workload("bf16_L8k_r0.5", 1, 32, 8, 8192, 128, 4096, 64, 4, "bf16"),
    "bf16_L32k_r0.25": Workload("bf16_L32k_r0.25", 1, 32, 8, 32768, 128, 8192, 64, 4, "bf16"),
    "bf16_L128k_r0.5": Workload("bf16_L128k_r0.5", 1, 32, 8, 131072, 128, _keep(0.5, 131072), 64, 4, "bf16"),
    "bf16_L128k_r0.25": Workload("bf16_L128k_r0.25", 1, 32, 8, 131072, 128, _keep(0.25, 131072), 64, 4, "bf16"),
    "bf16_L128k_r0.1": Workload("bf16_L128k_r0.1", 1, 32, 8, 131072, 128, _keep(0.1, 131072), 64, 4, "bf16"),
    # Skewed importance: 1% planted keys per KV head, two batch entries.
    "bf16_L64k_planted": Workload("bf16_L64k_planted", 2, 32, 8, 65536, 128, _keep(0.1, 65536), 64, 4, "bf16",
                                  planted=True),
    # Adaptive budgets: token coverage 0.2, no cap below L, heads graded from diffuse to
    # concentrated (query scale 1 .. 4).
    "bf16_L128k_tau0.2_graded": Workload("bf16_L128k_tau0.2_graded", 1, 32, 8, 131072, 128, 131072, 64, 4, "bf16",
                                         tau=0.2, q_grade=4.0),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    u = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Raw bfloat16 bit patterns (uint16) of float32 values that are already bf16-exact."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw(tensor_id: int, shape, seed: int) -> np.ndarray:
    B, L = shape[0], shape[1]
    inner = int(np.prod(shape[2:]))
    out = np.empty((B, L, inner), dtype=np.float32)
    jobs = [(b, blk) for b in range(B) for blk in range((L + ROWS_PER_BLOCK - 1) // ROWS_PER_BLOCK)]

    def fill(job):
        b, blk = job
        p0 = blk * ROWS_PER_BLOCK
        p1 = min(L, p0 + ROWS_PER_BLOCK)
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tensor_id, b, blk)))
        out[b, p0:p1] = rng.standard_normal((p1 - p0, inner), dtype=np.float32)

    if len(jobs) == 1:
        fill(jobs[0])
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, jobs))
    return out.reshape(shape)


def plant_positions(w: Workload, b: int, g: int) -> np.ndarray:
    """Positions (sorted) whose keys are planted for batch entry b and KV head g."""
    n = int(round(PLANT_FRACTION * w.L))
    lo, hi = w.n_sink, w.L - w.W
    rng = np.random.default_rng(np.random.SeedSequence(w.seed, spawn_key=(4, b, g)))
    return np.sort(rng.choice(np.arange(lo, hi), size=n, replace=False))


def make_inputs(w: Workload) -> dict:
    """Draw the seeded inputs of workload ``w``.

    Returns float32 arrays ``q, k, v, r`` holding exactly the values of the storage dtype
    (bf16-rounded for bf16 workloads), and ``planted`` (dict (b, g) -> positions) when
    the workload plants keys.
    """
    q = _draw(0, (w.B, w.L, w.H, w.d), w.seed)
    if w.q_grade != 1.0 and w.H > 1:
        q *= (1.0 + (w.q_grade - 1.0) * np.arange(w.H, dtype=np.float32) / (w.H - 1))[None, None, :, None]
    k = _draw(1, (w.B, w.L, w.Hkv, w.d), w.seed)
    v = _draw(2, (w.B, w.L, w.Hkv, w.d), w.seed)
    r = _draw(3, (w.B, w.L, w.H, w.d), w.seed)
    if w.dtype == "bf16":
        q, k, v, r = (round_bf16(t) for t in (q, k, v, r))
    planted = {}
    if w.planted:
        G = w.G
        nq = min(PLANT_QUERY_ROWS, w.L)
        for b in range(w.B):
            for g in range(w.Hkv):
                pos = plant_positions(w, b, g)
                m = q[b, w.L - nq:, g * G:(g + 1) * G, :].astype(np.float64).reshape(-1, w.d).mean(axis=0)
                u = m / np.linalg.norm(m)
                norms = np.linalg.norm(k[b, pos, g, :].astype(np.float64), axis=-1, keepdims=True)
                newk = (PLANT_SCALE * norms * u[None, :]).astype(np.float32)
                k[b, pos, g, :] = round_bf16(newk) if w.dtype == "bf16" else newk
                planted[(b, g)] = pos
    return {"q": q, "k": k, "v": v, "r": r, "planted": planted}


def small_random(B, H, Hkv, L, d, seed=0, dtype="fp32", q_grade=1.0) -> dict:
    """Small seeded inputs of any shape (test cases); same recipe as ``make_inputs``."""
    w = Workload("adhoc", B, H, Hkv, L, d, L, 1, 0, dtype, seed=seed, q_grade=q_grade)
    return make_inputs(w)
