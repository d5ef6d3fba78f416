"""Token Sparse Attention on MI355X (gfx950): Python binding of libtsa.so.

Argument marshalling only.  Every stage runs in the library's HIP kernels; PyTorch
provides device memory and the current stream.  The functions named like the C entry
points (``tsa_score`` ... ``tsa_dense_attn``) take every buffer explicitly; the
lower-case helpers below them allocate outputs and workspace with torch and call them.

Layouts (contiguous): q, residual, out ``[B, L, H, d]``; k, v ``[B, L, Hkv, d]``;
scores ``[B, H, L]`` fp32; idx ``[B, R, keep]`` int32 ascending; compact qh, oh
``[B, H, keep, d]`` and kh, vh ``[B, R, keep, d]``, where R = H (one token subset per
query head) or R = Hkv (``per_kv_head=True``: the query heads of a KV head share one
subset chosen on their summed scores).  dtypes: float32 or bfloat16, head dim 64 or 128.

The library must have been built (``token_sparse_attention_head_amd/build.py``);
importing this package without it raises ImportError: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtsa.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "tsa.h")

TSA_OK = 0
TSA_F32, TSA_BF16 = 0, 1
TSA_OP_SCORE, TSA_OP_SELECT, TSA_OP_SCATTER, TSA_OP_FORWARD, TSA_OP_DRIFT = 0, 1, 2, 3, 4
TSA_SUBSETS_PER_HEAD, TSA_SUBSETS_PER_KV_HEAD = 0, 1
ABI_VERSION = 3   # TSA_ABI_VERSION of include/tsa.h that this binding's TsaDesc matches
STATUS_NAMES = {0: "TSA_OK", 1: "TSA_ERR_NULL", 2: "TSA_ERR_SHAPE", 3: "TSA_ERR_BUDGET", 4: "TSA_ERR_DTYPE",
                5: "TSA_ERR_ALIGN", 6: "TSA_ERR_WORKSPACE", 7: "TSA_ERR_ALIAS", 8: "TSA_ERR_LAUNCH", 9: "TSA_ERR_ARG"}


class TsaDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("L", ctypes.c_int32),
                ("d", ctypes.c_int32), ("keep", ctypes.c_int32), ("W", ctypes.c_int32), ("n_sink", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("subsets", ctypes.c_int32),
                ("tau", ctypes.c_float)]

    def __repr__(self):
        return "TsaDesc(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class TsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({lib().tsa_status_str(status).decode()})")


_LIB = None
_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_DP = ctypes.POINTER(TsaDesc)
_SIGS = {
    "tsa_abi_version": ([], ctypes.c_int),
    "tsa_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "tsa_check": ([_DP], ctypes.c_int),
    "tsa_workspace_size": ([_DP, ctypes.c_int, ctypes.POINTER(_SZ)], ctypes.c_int),
    "tsa_score": ([_DP, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "tsa_select": ([_DP, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "tsa_budget": ([_DP, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "tsa_gather_qkv": ([_DP, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "tsa_attn": ([_DP, _P, _P, _P, _P, _P], ctypes.c_int),
    "tsa_scatter_residual": ([_DP, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "tsa_forward": ([_DP, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "tsa_dense_attn": ([_DP, _P, _P, _P, _P, _P], ctypes.c_int),
    "tsa_drift": ([_DP, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
}


def lib():
    """The loaded libtsa.so (torch is imported first, so the library binds to torch's HIP runtime)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libtsa.so not built at {LIB_PATH}; run token_sparse_attention_head_amd/build.py")
        h = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        if h.tsa_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} has ABI version {h.tsa_abi_version()}, the binding expects {ABI_VERSION}; "
                              "rebuild it with token_sparse_attention_head_amd/build.py")
        _LIB = h
    return _LIB


def header_functions() -> list[str]:
    """Entry points declared in include/tsa.h."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:tsa_status|int|const char\*)\s+(tsa_\w+)\s*\(", text, re.M)))


# ---- descriptors and marshalling ------------------------------------------------------

def make_desc(B, H, Hkv, L, d, keep, W, n_sink, dtype, scale: float = 0.0, subsets: int = 0,
              tau: float = 0.0) -> TsaDesc:
    code = {torch.float32: TSA_F32, torch.bfloat16: TSA_BF16}.get(dtype, dtype)
    return TsaDesc(int(B), int(H), int(Hkv), int(L), int(d), int(keep), int(W), int(n_sink), int(code), float(scale),
                   int(subsets), float(tau))


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != TSA_OK:
        raise TsaError(st, name)


def tsa_check(desc: TsaDesc) -> int:
    return lib().tsa_check(ctypes.byref(desc))


def tsa_workspace_size(desc: TsaDesc, op: int) -> int:
    out = _SZ(0)
    _call("tsa_workspace_size", ctypes.byref(desc), int(op), ctypes.byref(out))
    return out.value


def tsa_score(desc, q, k, scores, ws, ws_bytes=None, stream=None):
    _call("tsa_score", ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(scores), _ptr(ws),
          ws.numel() if ws_bytes is None else ws_bytes, _stream(stream))


def tsa_select(desc, scores, idx, ws=None, ws_bytes=0, stream=None):
    _call("tsa_select", ctypes.byref(desc), _ptr(scores), _ptr(idx), _ptr(ws), ws_bytes, _stream(stream))


def tsa_budget(desc, scores, counts, ws=None, ws_bytes=0, stream=None):
    _call("tsa_budget", ctypes.byref(desc), _ptr(scores), _ptr(counts), _ptr(ws), ws_bytes, _stream(stream))


def tsa_gather_qkv(desc, q, k, v, idx, qh, kh, vh, stream=None):
    _call("tsa_gather_qkv", ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(qh), _ptr(kh), _ptr(vh),
          _stream(stream))


def tsa_attn(desc, qh, kh, vh, oh, stream=None):
    _call("tsa_attn", ctypes.byref(desc), _ptr(qh), _ptr(kh), _ptr(vh), _ptr(oh), _stream(stream))


def tsa_scatter_residual(desc, oh, idx, residual, out, ws=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel()
    _call("tsa_scatter_residual", ctypes.byref(desc), _ptr(oh), _ptr(idx), _ptr(residual), _ptr(out), _ptr(ws),
          ws_bytes, _stream(stream))


def tsa_forward(desc, q, k, v, residual, out, scores=None, idx=None, ws=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel()
    _call("tsa_forward", ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(residual), _ptr(out), _ptr(scores),
          _ptr(idx), _ptr(ws), ws_bytes, _stream(stream))


def tsa_dense_attn(desc, q, k, v, o, stream=None):
    _call("tsa_dense_attn", ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _stream(stream))


def tsa_drift(desc, a, b, out, ws, ws_bytes=None, stream=None):
    _call("tsa_drift", ctypes.byref(desc), _ptr(a), _ptr(b), _ptr(out), _ptr(ws),
          ws.numel() if ws_bytes is None else ws_bytes, _stream(stream))


# ---- allocating helpers ---------------------------------------------------------------

def _check_io(q, k, v=None):
    for t in (q, k, v):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("dtype must be float32 or bfloat16")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, L, H, d] and k, v [B, L, Hkv, d]")


def desc_for(q, k, keep, W=64, n_sink=4, scale=0.0, per_kv_head=False, tau=0.0) -> TsaDesc:
    B, L, H, d = q.shape
    keep = min(int(keep), L)   # a budget larger than the sequence keeps everything
    return make_desc(B, H, k.shape[2], L, d, keep, W, n_sink, q.dtype, scale,
                     TSA_SUBSETS_PER_KV_HEAD if per_kv_head else TSA_SUBSETS_PER_HEAD, tau)


def _workspace(desc, op, device):
    n = tsa_workspace_size(desc, op)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def score(q, k, W=64, scale=0.0):
    """Scores [B, H, L] (fp32) of every key, from the last W causal query rows of each head."""
    _check_io(q, k)
    desc = desc_for(q, k, q.shape[1], W, 0, scale)
    scores = torch.empty(q.shape[0], q.shape[2], q.shape[1], dtype=torch.float32, device=q.device)
    tsa_score(desc, q, k, scores, _workspace(desc, TSA_OP_SCORE, q.device))
    return scores


def _select_desc(scores, keep, W, n_sink, kv_heads, tau):
    if not scores.is_cuda or scores.dtype != torch.float32 or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous float32 GPU tensor")
    B, H, L = scores.shape
    R = H if kv_heads is None else int(kv_heads)
    return make_desc(B, H, R, L, 128, min(int(keep), L), W, n_sink, TSA_F32, 0.0,
                     TSA_SUBSETS_PER_HEAD if kv_heads is None else TSA_SUBSETS_PER_KV_HEAD, tau), R


def select(scores, keep, W=64, n_sink=4, kv_heads=None, tau=0.0):
    """idx [B, R, keep] (int32, ascending) from scores [B, H, L]: one subset per query head
    (R = H), or with kv_heads=Hkv one per KV head on the summed scores of its heads.  With
    tau > 0 each row holds its adaptive budget of positions, then -1 padding."""
    desc, R = _select_desc(scores, keep, W, n_sink, kv_heads, tau)
    idx = torch.empty(desc.B, R, desc.keep, dtype=torch.int32, device=scores.device)
    ws = _workspace(desc, TSA_OP_SELECT, scores.device)
    tsa_select(desc, scores, idx, ws, ws.numel())
    return idx


def budget(scores, keep, W=64, n_sink=4, kv_heads=None, tau=0.0):
    """counts [B, R] (int32): the positions each subset row keeps under token coverage tau
    (capped at keep; keep everywhere when tau = 0)."""
    desc, R = _select_desc(scores, keep, W, n_sink, kv_heads, tau)
    counts = torch.empty(desc.B, R, dtype=torch.int32, device=scores.device)
    ws = _workspace(desc, TSA_OP_SELECT, scores.device)
    tsa_budget(desc, scores, counts, ws, ws.numel())
    return counts


def gather_qkv(q, k, v, idx):
    """qh [B, H, keep, d], kh, vh [B, R, keep, d] from idx [B, R, keep] (R = H or Hkv)."""
    _check_io(q, k, v)
    B, L, H, d = q.shape
    R = idx.shape[1]
    if R not in (H, k.shape[2]) or idx.shape[0] != B:
        raise ValueError(f"idx must be [B, H, keep] or [B, Hkv, keep]; got {tuple(idx.shape)}")
    desc = desc_for(q, k, idx.shape[2], W=1, n_sink=0, per_kv_head=R != H)
    qh = torch.empty(B, H, idx.shape[2], d, dtype=q.dtype, device=q.device)
    kh, vh = (torch.empty(B, R, idx.shape[2], d, dtype=q.dtype, device=q.device) for _ in range(2))
    tsa_gather_qkv(desc, q, k, v, idx, qh, kh, vh)
    return qh, kh, vh


def attn(qh, kh, vh, scale=0.0):
    """Causal attention over the compact rows of every (batch, head): qh [B, H, keep, d],
    kh, vh [B, R, keep, d] (query head h uses row block h / (H / R))."""
    B, H, n, d = qh.shape
    R = kh.shape[1]
    desc = make_desc(B, H, R, n, d, n, 1, 0, qh.dtype, scale,
                     TSA_SUBSETS_PER_KV_HEAD if R != H else TSA_SUBSETS_PER_HEAD)
    oh = torch.empty_like(qh)
    tsa_attn(desc, qh, kh, vh, oh)
    return oh


def scatter_residual(oh, idx, residual, out=None):
    """out = residual + scatter(oh at idx); out=residual updates in place."""
    B, L, H, d = residual.shape
    R = idx.shape[1]
    desc = make_desc(B, H, R, L, d, idx.shape[2], 1, 0, residual.dtype, 0.0,
                     TSA_SUBSETS_PER_KV_HEAD if R != H else TSA_SUBSETS_PER_HEAD)
    if out is None:
        out = torch.empty_like(residual)
    ws = None if out.data_ptr() == residual.data_ptr() else _workspace(desc, TSA_OP_SCATTER, residual.device)
    tsa_scatter_residual(desc, oh, idx, residual, out, ws)
    return out


def forward(q, k, v, residual, keep, W=64, n_sink=4, scale=0.0, out=None, return_scores=False, ws=None,
            per_kv_head=False, tau=0.0):
    """One token-sparse attention layer: returns out (and scores [B, H, L], idx [B, R, keep]
    when asked).  tau > 0: adaptive budgets capped at keep."""
    _check_io(q, k, v)
    desc = desc_for(q, k, keep, W, n_sink, scale, per_kv_head, tau)
    if out is None:
        out = torch.empty_like(residual)
    if ws is None:
        ws = _workspace(desc, TSA_OP_FORWARD, q.device)
    scores = idx = None
    if return_scores:
        B, L, H, _ = q.shape
        scores = torch.empty(B, H, L, dtype=torch.float32, device=q.device)
        idx = torch.empty(B, k.shape[2] if per_kv_head else H, desc.keep, dtype=torch.int32, device=q.device)
    tsa_forward(desc, q, k, v, residual, out, scores, idx, ws)
    return (out, scores, idx) if return_scores else out


def dense_attn(q, k, v, scale=0.0):
    """Dense causal attention [B, L, H, d] with grouped-query heads (the library's reference)."""
    _check_io(q, k, v)
    desc = desc_for(q, k, q.shape[1], 1, 0, scale)
    o = torch.empty_like(q)
    tsa_dense_attn(desc, q, k, v, o)
    return o


def drift(h_before, h_after):
    """Representation drift (a 0-dim float64 GPU tensor) of hidden states [B, L, D] or
    [B, L, H, d] (D = H * d a multiple of 64): 1 - mean over tokens of the cosine of the
    normalised before/after vectors."""
    if h_before.shape != h_after.shape or h_before.dtype != h_after.dtype:
        raise ValueError("hidden states must have the same shape and dtype")
    for t in (h_before, h_after):
        if not t.is_cuda or not t.is_contiguous() or t.dtype not in (torch.float32, torch.bfloat16) or t.dim() < 3:
            raise ValueError("hidden states must be contiguous float32/bfloat16 GPU tensors [B, L, ...]")
    B, L = h_before.shape[0], h_before.shape[1]
    D = h_before[0, 0].numel()
    d = 128 if D % 128 == 0 else 64
    if D % d:
        raise ValueError("the hidden size must be a multiple of 64")
    desc = make_desc(B, D // d, D // d, L, d, 0, 1, 0, h_before.dtype)
    out = torch.empty((), dtype=torch.float64, device=h_before.device)
    ws = _workspace(desc, TSA_OP_DRIFT, h_before.device)
    tsa_drift(desc, h_before, h_after, out, ws)
    return out


class LayerStability:
    """Host-side stability rule over per-layer drifts: a layer is stable once the mean of
    the last ``window`` drifts (its own included) is below ``threshold``."""

    def __init__(self, window: int = 3, threshold: float = 0.1):
        self.window, self.threshold, self.history = window, threshold, []

    def update(self, drift_value: float) -> bool:
        self.history.append(float(drift_value))
        if len(self.history) < self.window:
            return False
        recent = self.history[-self.window:]
        return sum(recent) / len(recent) < self.threshold
