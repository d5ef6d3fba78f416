"""Oracle for Token Sparse Attention's per-layer path: plain, slow, float64, CPU only.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module.  It shares no code with the HIP library and imports
nothing from it; the two meet only through the seeded inputs of ``workloads.py``.

What it computes, stage by stage, in the order the method runs (sources: the skill page
"Token Sparse Attention Long Context", Steps 1-3, and the paper page "Token Sparse
Attention: Efficient Long-Context Inference with Interleaved Token Selection",
Figure 3 and the Abstract):

1. ``score``     -- per query head h, the causal softmax(q k^T / sqrt(d)) rows of the
                    last W query positions, summed over those rows: one importance
                    score per key position (skill page, Step 1, the query-key
                    alignment scorer, restricted to the last W causal rows).
2. ``select``    -- the per-head subset S_h: the first ``n_sink`` positions and the
                    last W positions always, plus the highest-scoring other positions
                    up to ``keep`` in total; equal scores go to the lower position;
                    S_h is returned in ascending position order (skill page, Step 1,
                    top-K selection; Figure 3's per-head subset).
3. ``gather``    -- Q^, K^, V^ = the rows of Q, K, V at S_h; query head h reads KV
                    head floor(h / G) (skill page, Step 2; Figure 3, stage 1).
4. ``attend``    -- dense causal softmax attention on the compact rows (skill page,
                    Step 3; Figure 3, stage 2; the Abstract's compatibility with dense
                    attention kernels).
5. ``scatter_residual`` -- the compact outputs put back at their positions, zero at
                    every other position, and the residual added everywhere (Figure 3:
                    scatter back to the full layout, then add the residual).

Subsets per KV head (``per_kv_head`` / ``kv_heads``): an extension of the library, not
from the pages, which define per-head subsets only.  The G query heads of KV head g share
one subset S_g, chosen by the same rule as a per-head subset but on ``group_scores``: the
sum of the G heads' score rows, taken in ascending head order in the scores' own dtype.
Every other stage is unchanged except that head h uses S_{h // G} and the compact K/V
rows are held once per subset.

Adaptive budgets (``tau`` / ``coverage_budget``): the paper page's TL;DR says per-head
sparsity budgets adapt on the fly through a dynamic token coverage, and its Figures 1 and
5 call tau the token coverage, a sparsity level where a higher value is sparser (0.005 in
Figure 5).  The pages give no formula, so the reading here is: a subset row drops its
lowest-scoring non-forced positions, one at a time in the reverse of the keep order,
while their scores add up to at most tau times the row's total score; the budget K_h is
what remains, capped at ``keep``.  Scores are counted in whole units of 2^-40 (each score
rounded down) so that the integer K_h is decided by exact integer sums.  Rows with
K_h < keep are padded with -1 in idx; gather gives zero rows there and scatter skips them.

Representation drift (``drift``, ``layer_stable``): the skill page's Step 4 measures how
much a layer changes the hidden states as one minus the mean, over tokens, of the cosine
between each token's normalised vector before and after the layer (each vector divided
by the larger of its norm and 1e-12), and calls a layer stable once the mean of its last
three drifts is below 0.1.

Every function works in float64; bf16 and fp32 inputs widen to float64 exactly.
The readings taken where the pages are silent (window, causality, ties, order, the
residual everywhere, the GQA head map, scale 1/sqrt(head_dim)) are stated at each
function.  Non-finite inputs are rejected.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "window", "forced_positions", "score", "score_head", "select", "select_row",
    "gather", "attend", "attend_rows", "scatter_residual", "forward", "threshold", "group_scores",
    "MASS_UNIT_BITS", "mass_units", "coverage_budget_row", "coverage_budget",
    "NORMALIZE_EPS", "drift", "layer_stable",
]


def _f64(x) -> np.ndarray:
    a = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(a)):
        raise ValueError("oracle inputs must be finite")
    return a


def window(L: int, W: int) -> int:
    """Number of scoring query rows: the last W positions, clipped to the sequence."""
    return min(W, L)


def forced_positions(L: int, W: int, n_sink: int) -> np.ndarray:
    """Positions every head keeps: sinks [0, n_sink) and the window [L-W, L), as a set
    union clipped to [0, L), ascending."""
    Wp = window(L, W)
    f = set(range(min(n_sink, L))) | set(range(L - Wp, L))
    return np.array(sorted(f), dtype=np.int64)


def score_head(qh: np.ndarray, kg: np.ndarray, W: int, scale: float) -> np.ndarray:
    """Scores of one (batch, query head): qh [L,d], kg [L,d] (its KV head) -> [L].

    Row i in [L-W', L) gives z_ij = scale * <q_i, k_j> for j <= i and the softmax over
    those j; the score of key j is the sum of its weights over the rows (skill page,
    Step 1: softmax along keys, summed along queries, logits divided by sqrt(d)).
    """
    L = qh.shape[0]
    Wp = window(L, W)
    rows = np.arange(L - Wp, L)
    z = scale * (qh[rows] @ kg.T)                       # [W', L]
    z[np.arange(L)[None, :] > rows[:, None]] = -np.inf   # causal: key j visible to row i iff j <= i
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    return p.sum(axis=0)


def score(q, k, W: int, scale: float | None = None) -> np.ndarray:
    """Scores for all heads: q [B,L,H,d], k [B,L,Hkv,d] -> s [B,H,L] (float64).

    Query head h uses KV head floor(h / G), G = H / Hkv (consecutive query heads share a
    KV head)."""
    q, k = _f64(q), _f64(k)
    B, L, H, d = q.shape
    Hkv = k.shape[2]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    G = H // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    s = np.empty((B, H, L), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s[b, h] = score_head(q[b, :, h, :], k[b, :, h // G, :], W, scale)
    return s


def select_row(s_row, keep: int, W: int, n_sink: int) -> np.ndarray:
    """S_h for one head from its scores [L]: forced positions, then the best other
    positions by (higher score, then lower position) until ``keep`` are held; returned
    ascending (skill page, Step 1, top-K selection)."""
    s_row = np.asarray(s_row, dtype=np.float64)
    L = s_row.shape[0]
    F = forced_positions(L, W, n_sink)
    if not (len(F) <= keep <= L):
        raise ValueError(f"keep={keep} outside [{len(F)}, {L}]")
    is_forced = np.zeros(L, dtype=bool)
    is_forced[F] = True
    cand = np.nonzero(~is_forced)[0]
    order = np.lexsort((cand, -s_row[cand]))   # primary: score descending; secondary: position ascending
    chosen = cand[order[: keep - len(F)]]
    return np.sort(np.concatenate([F, chosen]))


def group_scores(s, kv_heads: int) -> np.ndarray:
    """[B,H,L] -> [B,kv_heads,L]: row g is the sum of the score rows of query heads
    g*G .. g*G+G-1, added one head at a time in ascending order, in the dtype of ``s``
    (a float32 input is summed in float32, as the kernel does, so the two rank the
    positions identically)."""
    s = np.asarray(s)
    B, H, L = s.shape
    G = H // kv_heads
    out = np.empty((B, kv_heads, L), dtype=s.dtype)
    for g in range(kv_heads):
        acc = s[:, g * G, :].copy()
        for j in range(1, G):
            acc = acc + s[:, g * G + j, :]
        out[:, g, :] = acc
    return out


MASS_UNIT_BITS = 40


def mass_units(s_row) -> list:
    """Each score as a whole number of 2^-40 units, rounded down (Python integers; exact,
    since multiplying a float by 2^40 only moves its exponent)."""
    return [int(math.floor(float(x) * 2.0 ** MASS_UNIT_BITS)) for x in np.asarray(s_row, dtype=np.float64)]


def coverage_budget_row(s_row, keep: int, W: int, n_sink: int, tau: float) -> int:
    """K_h of one subset row under token coverage tau (paper page: TL;DR, Figures 1 and 5;
    the rule is this library's reading, stated in the module docstring).

    Mass budget: floor(tau * total), with tau taken as a float32 value and the product
    formed in float64, total = the sum of all L scores in units.  Positions leave in the
    reverse of the keep order (lower score first, among equal scores the higher position
    first) while the mass that left stays within the budget; forced positions never leave.
    """
    units = mass_units(s_row)
    L = len(units)
    F = forced_positions(L, W, n_sink)
    if not (len(F) <= keep <= L):
        raise ValueError(f"keep={keep} outside [{len(F)}, {L}]")
    s_row = np.asarray(s_row, dtype=np.float64)
    budget = int(math.floor(float(np.float32(tau)) * float(sum(units))))
    is_forced = np.zeros(L, dtype=bool)
    is_forced[F] = True
    cand = np.nonzero(~is_forced)[0]
    leave_order = cand[np.lexsort((-cand, s_row[cand]))]   # primary: score ascending; then position descending
    spent, left = 0, 0
    for j in leave_order:
        if spent + units[j] > budget:
            break
        spent += units[j]
        left += 1
    return min(L - left, keep)


def coverage_budget(s, keep: int, W: int, n_sink: int, tau: float, kv_heads: int | None = None) -> np.ndarray:
    """K_h for every subset row: [B,H,L] scores -> [B,R] int64 (R = H, or ``kv_heads``
    rows of ``group_scores``)."""
    if kv_heads is not None:
        s = group_scores(s, kv_heads)
    B, R, _ = np.asarray(s).shape
    out = np.empty((B, R), dtype=np.int64)
    for b in range(B):
        for r in range(R):
            out[b, r] = coverage_budget_row(s[b, r], keep, W, n_sink, tau)
    return out


def select(s, keep: int, W: int, n_sink: int, kv_heads: int | None = None, tau: float | None = None) -> np.ndarray:
    """idx [B,R,keep] (int64, strictly ascending per subset) from scores [B,H,L]: one
    subset per query head (R = H), or with ``kv_heads`` one per KV head on
    ``group_scores`` (R = kv_heads).  With ``tau`` > 0 row r holds its K_r =
    ``coverage_budget`` positions, then -1 up to ``keep``."""
    if kv_heads is not None:
        s = group_scores(s, kv_heads)
    B, R, _ = np.asarray(s).shape
    counts = coverage_budget(s, keep, W, n_sink, tau) if tau else None
    s = np.asarray(s, dtype=np.float64)
    idx = np.full((B, R, keep), -1, dtype=np.int64)
    for b in range(B):
        for r in range(R):
            kr = keep if counts is None else int(counts[b, r])
            idx[b, r, :kr] = select_row(s[b, r], kr, W, n_sink)
    return idx


def threshold(s_row, keep: int, W: int, n_sink: int) -> float:
    """The score of the last non-forced position taken (the (keep-|F|)-th best), or +inf
    when no non-forced position is taken."""
    s_row = np.asarray(s_row, dtype=np.float64)
    L = s_row.shape[0]
    F = forced_positions(L, W, n_sink)
    n = keep - len(F)
    if n <= 0:
        return float("inf")
    mask = np.ones(L, dtype=bool)
    mask[F] = False
    return float(np.sort(s_row[mask])[::-1][n - 1])


def gather(q, k, v, idx):
    """Q^[b,h,t] = Q[b,S_t,h]; K^[b,r,t] = K[b,S_t,g]; V^[b,r,t] = V[b,S_t,g], where
    query head h uses subset r = h // (H/R) and g = h // G is its KV head (skill page,
    Step 2, gather by index; Figure 3, stage 1).  idx [B,R,keep] -> Q^ [B,H,keep,d],
    K^, V^ [B,R,keep,d] (R = H: per head, one copy of the K/V rows per query head).
    Padding entries (-1) give zero rows."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, L, H, d = q.shape
    G = H // k.shape[2]
    R, keep = idx.shape[1], idx.shape[2]
    SG = H // R
    qh = np.empty((B, H, keep, d))
    kh = np.empty((B, R, keep, d))
    vh = np.empty((B, R, keep, d))
    valid = (idx >= 0)[..., None]
    safe = np.where(idx >= 0, idx, 0)
    for b in range(B):
        for h in range(H):
            qh[b, h] = np.where(valid[b, h // SG], q[b, safe[b, h // SG], h, :], 0.0)
        for r in range(R):
            g = (r * SG) // G
            kh[b, r] = np.where(valid[b, r], k[b, safe[b, r], g, :], 0.0)
            vh[b, r] = np.where(valid[b, r], v[b, safe[b, r], g, :], 0.0)
    return qh, kh, vh


def _attend_head(qh, kh, vh, scale, rows):
    out = np.empty((len(rows), qh.shape[1]))
    # Causal softmax attention, a block of query rows at a time (never a full keep x keep matrix).
    blk = 128
    for a in range(0, len(rows), blk):
        rr = rows[a:a + blk]
        hi = int(rr.max()) + 1
        z = scale * (qh[rr] @ kh[:hi].T)                         # [nr, hi]
        z[np.arange(hi)[None, :] > rr[:, None]] = -np.inf        # compact position u visible to t iff u <= t
        z -= z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p /= p.sum(axis=1, keepdims=True)
        out[a:a + len(rr)] = p @ vh[:hi]
    return out


def attend(qh, kh, vh, scale: float | None = None) -> np.ndarray:
    """O^[b,h,t] = sum over u <= t of softmax_u(scale <Q^_t, K^_u>) V^_u (skill page,
    Step 3; Figure 3, stage 2).  Causality on compact positions equals causality on the
    original positions because S_h is ascending."""
    qh, kh, vh = _f64(qh), _f64(kh), _f64(vh)
    B, H, n, d = qh.shape
    SG = H // kh.shape[1]                     # query heads per K^/V^ row block
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    oh = np.empty_like(qh)
    rows = np.arange(n)
    for b in range(B):
        for h in range(H):
            oh[b, h] = _attend_head(qh[b, h], kh[b, h // SG], vh[b, h // SG], scale, rows)
    return oh


def attend_rows(qh_bh, kh_bh, vh_bh, rows, scale: float) -> np.ndarray:
    """Compact attention of one (batch, head) at the given compact rows only -> [len(rows), d]."""
    return _attend_head(_f64(qh_bh), _f64(kh_bh), _f64(vh_bh), float(scale), np.asarray(rows, dtype=np.int64))


def scatter_residual(oh, idx, r) -> np.ndarray:
    """Out[b,p,h] = R[b,p,h] + O^[b,h,rank(p)] if p is in S_h, else R[b,p,h] (the compact
    outputs scattered into a zero full-length tensor, then the residual added: Figure 3,
    stage 2; skill page, Step 2).  Padding entries (-1) of idx are skipped."""
    oh, r = _f64(oh), _f64(r)
    out = r.copy()
    B, H, n, _ = oh.shape
    SG = H // idx.shape[1]                    # query heads per subset
    for b in range(B):
        for h in range(H):
            row = idx[b, h // SG]
            ok = row >= 0
            out[b, row[ok], h, :] += oh[b, h][ok]
    return out


def forward(q, k, v, r, keep: int, W: int, n_sink: int, scale: float | None = None,
            per_kv_head: bool = False, tau: float | None = None) -> dict:
    """All five stages; returns scores, idx, the compact tensors, O^ and Out."""
    d = np.asarray(q).shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    s = score(q, k, W, scale)
    idx = select(s, keep, W, n_sink, np.asarray(k).shape[2] if per_kv_head else None, tau)
    qh, kh, vh = gather(q, k, v, idx)
    oh = attend(qh, kh, vh, scale)
    out = scatter_residual(oh, idx, r)
    return {"scores": s, "idx": idx, "qh": qh, "kh": kh, "vh": vh, "oh": oh, "out": out}


NORMALIZE_EPS = 1e-12


def drift(h_before, h_after) -> float:
    """1 - mean over tokens of <h_before_t / max(|h_before_t|, eps), h_after_t / max(|h_after_t|, eps)>
    for [..., dim] hidden states (skill page, Step 4, the representation drift)."""
    a = _f64(h_before)
    b = _f64(h_after)
    a = a.reshape(-1, a.shape[-1])
    b = b.reshape(-1, b.shape[-1])
    na = np.maximum(np.sqrt((a * a).sum(axis=1)), NORMALIZE_EPS)
    nb = np.maximum(np.sqrt((b * b).sum(axis=1)), NORMALIZE_EPS)
    cos = ((a / na[:, None]) * (b / nb[:, None])).sum(axis=1)
    return float(1.0 - cos.mean())


def layer_stable(drifts, window: int = 3, threshold: float = 0.1) -> list:
    """For a sequence of per-layer drifts, whether each layer counts as stable: the mean of
    the last ``window`` drifts seen so far (this one included) is below ``threshold``;
    never before ``window`` drifts have been seen (skill page, Step 4)."""
    out = []
    for i in range(len(drifts)):
        if i + 1 < window:
            out.append(False)
            continue
        recent = drifts[i + 1 - window:i + 1]
        out.append(sum(recent) / len(recent) < threshold)
    return out
