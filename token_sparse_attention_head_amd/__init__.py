"""Token Sparse Attention on MI355X (gfx950): Python binding of libtsa.so.

Argument marshalling only.  Every stage runs in the library's HIP kernels; PyTorch
provides device memory and the current stream.  The functions named like the C entry
points (``tsa_score`` ... ``tsa_dense_attn``) take every buffer explicitly and check each
tensor against the descriptor (bytes, dtype, contiguity, device) before the call, so a
mismatched buffer raises ValueError instead of reaching the library; the lower-case
helpers below them allocate outputs and workspace with torch and call them.

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
TSA_OP_SCORE, TSA_OP_SELECT, TSA_OP_SCATTER, TSA_OP_FORWARD, TSA_OP_DRIFT, TSA_OP_SPARSE_ATTN = 0, 1, 2, 3, 4, 5
TSA_SUBSETS_PER_HEAD, TSA_SUBSETS_PER_KV_HEAD = 0, 1
ABI_VERSION = 4   # TSA_ABI_VERSION of include/tsa.h that this binding's TsaDesc matches
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
    "tsa_sparse_attn": ([_DP, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "tsa_stream_copy": ([_P, _P, _SZ, _P], ctypes.c_int),
    "tsa_forward_noalloc": ([_DP, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
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


_TORCH_OF = {TSA_F32: torch.float32, TSA_BF16: torch.bfloat16}


def _rows(desc) -> int:
    """Subset rows R of a descriptor: H (one subset per query head) or Hkv (per KV head)."""
    return desc.Hkv if desc.subsets == TSA_SUBSETS_PER_KV_HEAD else desc.H


def _nbytes(desc):
    """Bytes of every buffer kind a descriptor implies (the layouts of include/tsa.h)."""
    e = 2 if desc.dtype == TSA_BF16 else 4
    B, H, Hkv, L, d, K, R = desc.B, desc.H, desc.Hkv, desc.L, desc.d, desc.keep, _rows(desc)
    return {"full": B * L * H * d * e, "kv": B * L * Hkv * d * e, "scores": B * H * L * 4, "idx": B * R * K * 4,
            "counts": B * R * 4, "qh": B * H * K * d * e, "kvh": B * R * K * d * e}


def _arg(t, desc, kind, name, dtype=None):
    """One argument, checked: a tensor must be contiguous and hold at least the bytes the
    descriptor implies for its kind, in the expected dtype (the descriptor's dtype unless
    `dtype` is given); an int is a raw device address taken as is.  Returns (value, name);
    _call checks the device of every tensor after all arguments passed these checks."""
    if t is None or isinstance(t, int):
        return (t, name)
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor or a device address")
    want = dtype if dtype is not None else _TORCH_OF.get(desc.dtype)
    if want is not None and t.dtype != want:
        raise ValueError(f"{name} must be {want}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    need = _nbytes(desc)[kind] if kind else 0
    if t.numel() * t.element_size() < need:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes; the descriptor needs {need}")
    return (t, name)


def _ws(ws, ws_bytes, name="ws"):
    """Workspace argument and size: ws_bytes defaults to the tensor's size and may not exceed it."""
    if ws is None or isinstance(ws, int):
        return (ws, name), int(ws_bytes or 0)
    if not isinstance(ws, torch.Tensor) or not ws.is_contiguous():
        raise ValueError(f"{name} must be a contiguous torch tensor")
    size = ws.numel() * ws.element_size()
    n = size if ws_bytes is None else int(ws_bytes)
    if n > size:
        raise ValueError(f"{name}_bytes = {n} exceeds the {size} bytes of {name}")
    return (ws, name), n


class _Stream:
    """A stream argument, resolved by _call after the buffer checks (None: torch's current
    stream, the one every library call then runs on)."""

    def __init__(self, stream):
        self.stream = stream

    def handle(self) -> int | None:
        if self.stream is None:
            return torch.cuda.current_stream().cuda_stream
        if isinstance(self.stream, int):
            return self.stream
        return self.stream.cuda_stream


def _stream(stream) -> _Stream:
    return _Stream(stream)


def _call(name, *args):
    """Calls entry point `name`; (value, name) pairs from _arg / _ws become device addresses
    once every tensor among them is found on a GPU."""
    conv = []
    for a in args:
        if isinstance(a, tuple):
            t, nm = a
            if isinstance(t, torch.Tensor):
                if not t.is_cuda:
                    raise ValueError(f"{nm} must be on a GPU device")
                t = t.data_ptr()
            a = t
        conv.append(a)
    conv = [a.handle() if isinstance(a, _Stream) else a for a in conv]
    st = getattr(lib(), name)(*conv)
    if st != TSA_OK:
        raise TsaError(st, name)


def tsa_check(desc: TsaDesc) -> int:
    return lib().tsa_check(ctypes.byref(desc))


def tsa_workspace_size(desc: TsaDesc, op: int) -> int:
    out = _SZ(0)
    _call("tsa_workspace_size", ctypes.byref(desc), int(op), ctypes.byref(out))
    return out.value


def tsa_score(desc, q, k, scores, ws, ws_bytes=None, stream=None):
    w, n = _ws(ws, ws_bytes)
    _call("tsa_score", ctypes.byref(desc), _arg(q, desc, "full", "q"), _arg(k, desc, "kv", "k"),
          _arg(scores, desc, "scores", "scores", torch.float32), w, n, _stream(stream))


def tsa_select(desc, scores, idx, ws=None, ws_bytes=None, stream=None):
    w, n = _ws(ws, ws_bytes)
    _call("tsa_select", ctypes.byref(desc), _arg(scores, desc, "scores", "scores", torch.float32),
          _arg(idx, desc, "idx", "idx", torch.int32), w, n, _stream(stream))


def tsa_budget(desc, scores, counts, ws=None, ws_bytes=None, stream=None):
    w, n = _ws(ws, ws_bytes)
    _call("tsa_budget", ctypes.byref(desc), _arg(scores, desc, "scores", "scores", torch.float32),
          _arg(counts, desc, "counts", "counts", torch.int32), w, n, _stream(stream))


def tsa_gather_qkv(desc, q, k, v, idx, qh, kh, vh, stream=None):
    _call("tsa_gather_qkv", ctypes.byref(desc), _arg(q, desc, "full", "q"), _arg(k, desc, "kv", "k"),
          _arg(v, desc, "kv", "v"), _arg(idx, desc, "idx", "idx", torch.int32), _arg(qh, desc, "qh", "qh"),
          _arg(kh, desc, "kvh", "kh"), _arg(vh, desc, "kvh", "vh"), _stream(stream))


def tsa_attn(desc, qh, kh, vh, oh, stream=None):
    _call("tsa_attn", ctypes.byref(desc), _arg(qh, desc, "qh", "qh"), _arg(kh, desc, "kvh", "kh"),
          _arg(vh, desc, "kvh", "vh"), _arg(oh, desc, "qh", "oh"), _stream(stream))


def tsa_scatter_residual(desc, oh, idx, residual, out, ws=None, ws_bytes=None, stream=None):
    w, n = _ws(ws, ws_bytes)
    _call("tsa_scatter_residual", ctypes.byref(desc), _arg(oh, desc, "qh", "oh"),
          _arg(idx, desc, "idx", "idx", torch.int32), _arg(residual, desc, "full", "residual"),
          _arg(out, desc, "full", "out"), w, n, _stream(stream))


def tsa_forward(desc, q, k, v, residual, out, scores=None, idx=None, ws=None, ws_bytes=None, stream=None):
    w, n = _ws(ws, ws_bytes)
    _call("tsa_forward", ctypes.byref(desc), _arg(q, desc, "full", "q"), _arg(k, desc, "kv", "k"),
          _arg(v, desc, "kv", "v"), _arg(residual, desc, "full", "residual"), _arg(out, desc, "full", "out"),
          _arg(scores, desc, "scores", "scores", torch.float32), _arg(idx, desc, "idx", "idx", torch.int32), w, n,
          _stream(stream))


def tsa_forward_noalloc(desc, q, k, v, residual, out, scores, idx, stream=None):
    """tsa_forward on the library's static per-GPU scratch (no workspace; scores and idx required)."""
    _call("tsa_forward_noalloc", ctypes.byref(desc), _arg(q, desc, "full", "q"), _arg(k, desc, "kv", "k"),
          _arg(v, desc, "kv", "v"), _arg(residual, desc, "full", "residual"), _arg(out, desc, "full", "out"),
          _arg(scores, desc, "scores", "scores", torch.float32), _arg(idx, desc, "idx", "idx", torch.int32),
          _stream(stream))


def tsa_sparse_attn(desc, q, k, v, idx, residual, out, ws=None, ws_bytes=None, stream=None):
    w, n = _ws(ws, ws_bytes)
    _call("tsa_sparse_attn", ctypes.byref(desc), _arg(q, desc, "full", "q"), _arg(k, desc, "kv", "k"),
          _arg(v, desc, "kv", "v"), _arg(idx, desc, "idx", "idx", torch.int32),
          _arg(residual, desc, "full", "residual"), _arg(out, desc, "full", "out"), w, n, _stream(stream))


def tsa_dense_attn(desc, q, k, v, o, stream=None):
    _call("tsa_dense_attn", ctypes.byref(desc), _arg(q, desc, "full", "q"), _arg(k, desc, "kv", "k"),
          _arg(v, desc, "kv", "v"), _arg(o, desc, "full", "o"), _stream(stream))


def tsa_drift(desc, a, b, out, ws, ws_bytes=None, stream=None):
    w, n = _ws(ws, ws_bytes)
    _call("tsa_drift", ctypes.byref(desc), _arg(a, desc, "full", "a"), _arg(b, desc, "full", "b"),
          _arg(out, desc, None, "drift", torch.float64), w, n, _stream(stream))


def tsa_stream_copy(dst, src, nbytes=None, stream=None):
    """Plain device copy of nbytes (default: all of src) from src to dst."""
    for t, nm in ((dst, "dst"), (src, "src")):
        if not isinstance(t, int) and (not isinstance(t, torch.Tensor) or not t.is_contiguous()):
            raise ValueError(f"{nm} must be a contiguous torch tensor or a device address")
    size = lambda t: None if isinstance(t, int) else t.numel() * t.element_size()   # noqa: E731
    n = size(src) if nbytes is None else int(nbytes)
    for t, nm in ((dst, "dst"), (src, "src")):
        if size(t) is not None and size(t) < n:
            raise ValueError(f"{nm} holds fewer than {n} bytes")
        if isinstance(t, torch.Tensor) and not t.is_cuda:
            raise ValueError(f"{nm} must be on a GPU device")
    ptr = lambda t: t if isinstance(t, int) else t.data_ptr()   # noqa: E731
    _call("tsa_stream_copy", ptr(dst), ptr(src), n, _stream(stream))


# ---- allocating helpers ---------------------------------------------------------------

def _tensor(t, name, ndim, dtypes=(torch.float32, torch.bfloat16)):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _like(t, ref, name, ref_name):
    """t must have ref's shape and dtype."""
    if tuple(t.shape) != tuple(ref.shape):
        raise ValueError(f"{name} must have the shape of {ref_name} {tuple(ref.shape)}, got {tuple(t.shape)}")
    if t.dtype != ref.dtype:
        raise ValueError(f"{name} must have the dtype of {ref_name} ({ref.dtype}), got {t.dtype}")


def _same_gpu(*ts):
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError(f"tensors must be on one GPU device ({dev}, got {t.device})")


def _check_qkv(q, k, v=None):
    """q [B, L, H, d], k (and v) [B, L, Hkv, d] of one dtype, H a multiple of Hkv."""
    _tensor(q, "q", 4)
    _tensor(k, "k", 4)
    if k.dtype != q.dtype:
        raise ValueError(f"k must have the dtype of q ({q.dtype}), got {k.dtype}")
    B, L, H, d = q.shape
    if k.shape[0] != B or k.shape[1] != L or k.shape[3] != d or k.shape[2] < 1 or H % k.shape[2]:
        raise ValueError(f"k must be [B, L, Hkv, d] with H % Hkv == 0 for q {tuple(q.shape)}; got {tuple(k.shape)}")
    if v is not None:
        _tensor(v, "v", 4)
        _like(v, k, "v", "k")


def _check_idx(idx, B, heads, kv_heads):
    """idx int32 [B, R, keep] with R = H or R = Hkv; kv_heads None (not known to the caller):
    any R dividing H."""
    _tensor(idx, "idx", 3, (torch.int32,))
    R = idx.shape[1]
    ok = R in (heads, kv_heads) if kv_heads is not None else R >= 1 and heads % R == 0
    if idx.shape[0] != B or not ok:
        raise ValueError(f"idx must be int32 [B, H, keep] or [B, Hkv, keep] (B={B}, H={heads}, Hkv={kv_heads}); "
                         f"got {tuple(idx.shape)}")


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
    _check_qkv(q, k)
    _same_gpu(q, k)
    desc = desc_for(q, k, q.shape[1], W, 0, scale)
    scores = torch.empty(q.shape[0], q.shape[2], q.shape[1], dtype=torch.float32, device=q.device)
    tsa_score(desc, q, k, scores, _workspace(desc, TSA_OP_SCORE, q.device))
    return scores


def _select_desc(scores, keep, W, n_sink, kv_heads, tau):
    _tensor(scores, "scores", 3, (torch.float32,))
    B, H, L = scores.shape
    R = H if kv_heads is None else int(kv_heads)
    if R < 1 or H % R:
        raise ValueError(f"kv_heads must divide the {H} score rows per batch entry")
    _same_gpu(scores)
    return make_desc(B, H, R, L, 128, min(int(keep), L), W, n_sink, TSA_F32, 0.0,
                     TSA_SUBSETS_PER_HEAD if kv_heads is None else TSA_SUBSETS_PER_KV_HEAD, tau), R


def select(scores, keep, W=64, n_sink=4, kv_heads=None, tau=0.0):
    """idx [B, R, keep] (int32, ascending) from scores [B, H, L]: one subset per query head
    (R = H), or with kv_heads=Hkv one per KV head on the summed scores of its heads.  With
    tau > 0 each row holds its adaptive budget of positions, then -1 padding."""
    desc, R = _select_desc(scores, keep, W, n_sink, kv_heads, tau)
    idx = torch.empty(desc.B, R, desc.keep, dtype=torch.int32, device=scores.device)
    ws = _workspace(desc, TSA_OP_SELECT, scores.device)
    tsa_select(desc, scores, idx, ws)
    return idx


def budget(scores, keep, W=64, n_sink=4, kv_heads=None, tau=0.0):
    """counts [B, R] (int32): the positions each subset row keeps under token coverage tau
    (capped at keep; keep everywhere when tau = 0)."""
    desc, R = _select_desc(scores, keep, W, n_sink, kv_heads, tau)
    counts = torch.empty(desc.B, R, dtype=torch.int32, device=scores.device)
    ws = _workspace(desc, TSA_OP_SELECT, scores.device)
    tsa_budget(desc, scores, counts, ws)
    return counts


def gather_qkv(q, k, v, idx):
    """qh [B, H, keep, d], kh, vh [B, R, keep, d] from idx [B, R, keep] (R = H or Hkv)."""
    _check_qkv(q, k, v)
    B, L, H, d = q.shape
    _check_idx(idx, B, H, k.shape[2])
    _same_gpu(q, k, v, idx)
    R = idx.shape[1]
    desc = desc_for(q, k, idx.shape[2], W=1, n_sink=0, per_kv_head=R != H)
    qh = torch.empty(B, H, idx.shape[2], d, dtype=q.dtype, device=q.device)
    kh, vh = (torch.empty(B, R, idx.shape[2], d, dtype=q.dtype, device=q.device) for _ in range(2))
    tsa_gather_qkv(desc, q, k, v, idx, qh, kh, vh)
    return qh, kh, vh


def attn(qh, kh, vh, scale=0.0):
    """Causal attention over the compact rows of every (batch, head): qh [B, H, keep, d],
    kh, vh [B, R, keep, d] (query head h uses row block h / (H / R))."""
    _tensor(qh, "qh", 4)
    _tensor(kh, "kh", 4)
    _tensor(vh, "vh", 4)
    _like(vh, kh, "vh", "kh")
    B, H, n, d = qh.shape
    R = kh.shape[1]
    if kh.dtype != qh.dtype or kh.shape[0] != B or kh.shape[2] != n or kh.shape[3] != d or R < 1 or H % R:
        raise ValueError(f"kh, vh must be [B, R, keep, d] of qh's dtype with R dividing H for qh {tuple(qh.shape)}; "
                         f"got {tuple(kh.shape)} {kh.dtype}")
    _same_gpu(qh, kh, vh)
    desc = make_desc(B, H, R, n, d, n, 1, 0, qh.dtype, scale,
                     TSA_SUBSETS_PER_KV_HEAD if R != H else TSA_SUBSETS_PER_HEAD)
    oh = torch.empty_like(qh)
    tsa_attn(desc, qh, kh, vh, oh)
    return oh


def _check_out(out, residual):
    _tensor(out, "out", 4)
    _like(out, residual, "out", "residual")


def scatter_residual(oh, idx, residual, out=None):
    """out = residual + scatter(oh at idx); out=residual updates in place."""
    _tensor(residual, "residual", 4)
    B, L, H, d = residual.shape
    _check_idx(idx, B, H, None)
    R = idx.shape[1]
    _tensor(oh, "oh", 4)
    if tuple(oh.shape) != (B, H, idx.shape[2], d) or oh.dtype != residual.dtype:
        raise ValueError(f"oh must be [B, H, keep, d] = {(B, H, idx.shape[2], d)} of the residual's dtype; "
                         f"got {tuple(oh.shape)} {oh.dtype}")
    if out is not None:
        _check_out(out, residual)
    _same_gpu(residual, idx, oh, *([out] if out is not None else []))
    desc = make_desc(B, H, R, L, d, idx.shape[2], 1, 0, residual.dtype, 0.0,
                     TSA_SUBSETS_PER_KV_HEAD if R != H else TSA_SUBSETS_PER_HEAD)
    if out is None:
        out = torch.empty_like(residual, memory_format=torch.contiguous_format)
    ws = None if out.data_ptr() == residual.data_ptr() else _workspace(desc, TSA_OP_SCATTER, residual.device)
    tsa_scatter_residual(desc, oh, idx, residual, out, ws)
    return out


def _check_layer(q, k, v, residual, out, ws):
    _check_qkv(q, k, v)
    _tensor(residual, "residual", 4)
    _like(residual, q, "residual", "q")
    if out is not None:
        _check_out(out, residual)
    if ws is not None:
        _tensor(ws, "ws", 1, (torch.uint8,))
    return [q, k, v, residual] + [t for t in (out, ws) if t is not None]


def forward(q, k, v, residual, keep, W=64, n_sink=4, scale=0.0, out=None, return_scores=False, ws=None,
            per_kv_head=False, tau=0.0):
    """One token-sparse attention layer: returns out (and scores [B, H, L], idx [B, R, keep]
    when asked).  tau > 0: adaptive budgets capped at keep."""
    _same_gpu(*_check_layer(q, k, v, residual, out, ws))
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


def sparse_attn(q, k, v, idx, residual, out=None, scale=0.0, tau=0.0, ws=None):
    """Compress, attend and decompress on given subsets idx [B, R, keep] (as select writes
    them; R = H per head or Hkv per KV head): out = residual + scatter(attention of the
    gathered rows).  out=residual updates in place.  tau > 0 marks -1-padded rows."""
    ts = _check_layer(q, k, v, residual, out, ws)
    B, L, H, d = q.shape
    _check_idx(idx, B, H, k.shape[2])
    _same_gpu(*ts, idx)
    desc = desc_for(q, k, idx.shape[2], W=1, n_sink=0, scale=scale, per_kv_head=idx.shape[1] != H, tau=tau)
    if out is None:
        out = torch.empty_like(residual)
    if ws is None:
        ws = _workspace(desc, TSA_OP_SPARSE_ATTN, q.device)
    tsa_sparse_attn(desc, q, k, v, idx, residual, out, ws)
    return out


def dense_attn(q, k, v, scale=0.0):
    """Dense causal attention [B, L, H, d] with grouped-query heads (the library's reference)."""
    _check_qkv(q, k, v)
    _same_gpu(q, k, v)
    desc = desc_for(q, k, q.shape[1], 1, 0, scale)
    o = torch.empty_like(q)
    tsa_dense_attn(desc, q, k, v, o)
    return o


def drift(h_before, h_after):
    """Representation drift (a 0-dim float64 GPU tensor) of hidden states [B, L, D] or
    [B, L, H, d] (D = H * d a multiple of 64): 1 - mean over tokens of the cosine of the
    normalised before/after vectors."""
    for t, nm in ((h_before, "h_before"), (h_after, "h_after")):
        if not isinstance(t, torch.Tensor) or t.dim() < 3:
            raise ValueError(f"{nm} must be a tensor [B, L, ...]")
        _tensor(t, nm, t.dim())
    _like(h_after, h_before, "h_after", "h_before")
    _same_gpu(h_before, h_after)
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
