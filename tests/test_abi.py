"""C-ABI checks that need no GPU: the library loads, exports every entry point that
include/tsa.h declares, and rejects bad arguments on the host before launching anything.
Pointers here are fake addresses: validation fails before any memory is touched."""
import ctypes

import pytest

from tests._lib import ensure_built

tsa = ensure_built()
L = tsa.lib()

EXPECTED = ["tsa_abi_version", "tsa_attn", "tsa_budget", "tsa_check", "tsa_dense_attn", "tsa_drift",
            "tsa_forward", "tsa_forward_noalloc", "tsa_gather_qkv", "tsa_scatter_residual", "tsa_score", "tsa_select", "tsa_sparse_attn",
            "tsa_status_str", "tsa_stream_copy", "tsa_workspace_size"]


def D(**kw):
    base = dict(B=1, H=32, Hkv=8, L=8192, d=128, keep=4096, W=64, n_sink=4, dtype=tsa.TSA_BF16, scale=0.0,
                subsets=tsa.TSA_SUBSETS_PER_HEAD, tau=0.0)
    base.update(kw)
    return tsa.make_desc(**base)


def test_header_declares_and_library_exports_every_entry_point():
    declared = tsa.header_functions()
    assert declared == EXPECTED
    for name in declared:
        assert hasattr(L, name), name
    assert L.tsa_abi_version() == 4
    assert L.tsa_status_str(7) and L.tsa_status_str(1234) == b"unknown status"


@pytest.mark.parametrize("kw,code", [
    (dict(), 0),
    (dict(dtype=7), 4),
    (dict(H=0), 2), (dict(Hkv=3), 2), (dict(d=96), 2), (dict(L=-1), 2), (dict(B=-2), 2),
    (dict(keep=67), 3),            # |F| = 4 + 64 = 68
    (dict(keep=68), 0),
    (dict(keep=8193), 3),
    (dict(keep=8192), 0),
    (dict(W=0), 3), (dict(W=65), 3), (dict(n_sink=-1), 3),
    (dict(scale=-1.0), 9), (dict(scale=float("nan")), 9),
    (dict(L=40, keep=40, W=64), 0),            # window covers the whole sequence
    (dict(L=40, keep=39, W=64), 3),
    (dict(L=0, keep=0), 0),                    # empty problem: nothing to do
    (dict(B=0), 0),
    (dict(B=4096, H=32), 2),                   # grid limit
    # one batch entry's K below 4 GiB: L * Hkv * d * 2 < 2^32 (H = Hkv = 8, d = 128 bf16)
    (dict(H=8, Hkv=8, L=(1 << 21) - 64, keep=4096), 0),
    (dict(H=8, Hkv=8, L=1 << 21, keep=4096), 2),
    (dict(H=8, Hkv=8, L=1 << 20, keep=4096, dtype=0), 2),   # fp32: 4 bytes per element
    (dict(subsets=1), 0),                      # one subset per KV head
    (dict(subsets=2), 9), (dict(subsets=-1), 9),
    (dict(tau=0.005), 0), (dict(tau=1.0), 0),  # adaptive budgets
    (dict(tau=-0.1), 9), (dict(tau=1.5), 9), (dict(tau=float("nan")), 9),
])
def test_check_codes(kw, code):
    assert tsa.tsa_check(D(**kw)) == code


def test_workspace_sizes():
    d = D()
    # the select's radix histograms (2048 bins) and per-wave counts for each of the 32 rows
    assert 32 * 2048 * 4 <= tsa.tsa_workspace_size(d, tsa.TSA_OP_SELECT) < 32 * 8192 * 4
    assert tsa.tsa_workspace_size(d, tsa.TSA_OP_SCATTER) == 32 * 8192 * 4
    fwd = tsa.tsa_workspace_size(d, tsa.TSA_OP_FORWARD)
    # bf16 forward is fused: scores, idx and the inverse map, no compact tensors
    assert 2 * 32 * 8192 * 4 + 32 * 4096 * 4 <= fwd < 4 * 32 * 4096 * 128 * 2
    # fp32 forward runs the stages: four compact [B,H,keep,d] tensors as well
    fwd32 = tsa.tsa_workspace_size(D(dtype=tsa.TSA_F32), tsa.TSA_OP_FORWARD)
    assert fwd32 >= 4 * 32 * 4096 * 128 * 4 + 2 * 32 * 8192 * 4
    assert tsa.tsa_workspace_size(d, tsa.TSA_OP_SCORE) > 0
    with pytest.raises(tsa.TsaError) as e:
        tsa.tsa_workspace_size(d, 17)
    assert e.value.status == 9
    with pytest.raises(tsa.TsaError):
        tsa.tsa_workspace_size(D(keep=3), tsa.TSA_OP_FORWARD)
    # one subset per KV head: the select sums the 4 score rows of each group into [B, Hkv, L],
    # the inverse map has Hkv rows, and the staged fp32 forward holds K^/V^ per KV head only
    kv = D(subsets=tsa.TSA_SUBSETS_PER_KV_HEAD)
    assert 8 * 8192 * 4 + 8 * 2048 * 4 <= tsa.tsa_workspace_size(kv, tsa.TSA_OP_SELECT) < 2 * 8 * 8192 * 4
    assert tsa.tsa_workspace_size(kv, tsa.TSA_OP_SCATTER) == 8 * 8192 * 4
    kv32 = tsa.tsa_workspace_size(D(dtype=tsa.TSA_F32, subsets=1), tsa.TSA_OP_FORWARD)
    assert 2 * 32 * 4096 * 128 * 4 + 2 * 8 * 4096 * 128 * 4 <= kv32 < fwd32
    # adaptive budgets add 64-bit mass histograms to the select and the row budgets to the forward
    ad = D(tau=0.01)
    assert tsa.tsa_workspace_size(ad, tsa.TSA_OP_SELECT) >= tsa.tsa_workspace_size(d, tsa.TSA_OP_SELECT) + 32 * 2048 * 8
    assert tsa.tsa_workspace_size(ad, tsa.TSA_OP_FORWARD) > fwd
    # drift: partial sums only, sized by B*L; the budget fields are not looked at
    assert 0 < tsa.tsa_workspace_size(D(keep=3), tsa.TSA_OP_DRIFT) <= 2048 * 8
    assert tsa.tsa_workspace_size(D(L=0, keep=0), tsa.TSA_OP_DRIFT) == 0
    # sparse attention on given subsets: bf16 needs the inverse map only (plus row counts and
    # the per-XCD plan with adaptive budgets); fp32 also holds the four compact tensors
    assert tsa.tsa_workspace_size(d, tsa.TSA_OP_SPARSE_ATTN) == 32 * 8192 * 4
    assert tsa.tsa_workspace_size(ad, tsa.TSA_OP_SPARSE_ATTN) > 32 * 8192 * 4 + 32 * 4
    assert tsa.tsa_workspace_size(D(dtype=tsa.TSA_F32), tsa.TSA_OP_SPARSE_ATTN) >= 4 * 32 * 4096 * 128 * 4


A = 1 << 40           # fake, well-separated, 16-byte aligned addresses
GB = 1 << 32


def call(name, *args):
    return getattr(L, name)(*args)


def test_entry_points_reject_before_launch():
    d = D()
    bd = ctypes.byref(d)
    q, k, v, r, o = A, A + GB, A + 2 * GB, A + 3 * GB, A + 4 * GB
    qh, kh, vh, oh = A + 5 * GB, A + 6 * GB, A + 7 * GB, A + 8 * GB
    idx, sc, ws = A + 9 * GB, A + 10 * GB, A + 11 * GB
    big = 1 << 34
    # NULL pointers
    assert call("tsa_score", bd, None, k, sc, ws, big, None) == 1
    assert call("tsa_select", bd, sc, None, None, 0, None) == 1
    assert call("tsa_gather_qkv", bd, q, k, v, idx, qh, kh, None, None) == 1
    assert call("tsa_attn", bd, qh, kh, None, oh, None) == 1
    assert call("tsa_scatter_residual", bd, oh, idx, None, o, ws, big, None) == 1
    assert call("tsa_forward", bd, q, k, v, r, None, None, None, ws, big, None) == 1
    assert call("tsa_dense_attn", bd, q, k, v, None, None) == 1
    # misaligned
    assert call("tsa_gather_qkv", bd, q + 8, k, v, idx, qh, kh, vh, None) == 5
    assert call("tsa_attn", bd, qh, kh, vh, oh + 4, None) == 5
    assert call("tsa_forward", bd, q, k, v, r, o, sc + 2, None, ws, big, None) == 5
    # workspace
    assert call("tsa_score", bd, q, k, sc, ws, 16, None) == 6
    assert call("tsa_score", bd, q, k, sc, None, big, None) == 6
    assert call("tsa_scatter_residual", bd, oh, idx, r, o, ws, 16, None) == 6
    assert call("tsa_forward", bd, q, k, v, r, o, None, None, ws, 1024, None) == 6
    # aliasing
    assert call("tsa_gather_qkv", bd, q, k, v, idx, q + 4096, kh, vh, None) == 7
    assert call("tsa_gather_qkv", bd, q, k, v, idx, qh, qh + 4096, vh, None) == 7
    assert call("tsa_attn", bd, qh, kh, vh, qh, None) == 7
    assert call("tsa_scatter_residual", bd, oh, idx, r, r + 256, ws, big, None) == 7   # partial overlap
    assert call("tsa_scatter_residual", bd, oh, idx, r, oh, ws, big, None) == 7
    assert call("tsa_forward", bd, q, k, v, r, q, None, None, ws, big, None) == 7
    assert call("tsa_forward", bd, q, k, v, r, o, None, None, k, big, None) == 7
    assert call("tsa_dense_attn", bd, q, k, v, v, None) == 7
    assert call("tsa_score", bd, q, k, q, ws, big, None) == 7
    # the select always needs its workspace (per KV head it also holds the summed score rows)
    assert call("tsa_select", bd, sc, idx, None, 0, None) == 6
    assert call("tsa_select", bd, sc, idx, ws, 16, None) == 6
    assert call("tsa_select", bd, sc, idx, idx + 64, big, None) == 7
    assert call("tsa_budget", bd, sc, None, ws, big, None) == 1
    assert call("tsa_budget", bd, sc, idx, None, 0, None) == 6
    assert call("tsa_budget", bd, sc, idx + 4, ws, big, None) == 5
    assert call("tsa_budget", bd, sc, sc + 64, ws, big, None) == 7
    assert call("tsa_budget", bd, sc, idx, sc + 4096, big, None) == 7
    assert call("tsa_budget", ctypes.byref(D(tau=2.0)), sc, idx, ws, big, None) == 9
    kvd = ctypes.byref(D(subsets=tsa.TSA_SUBSETS_PER_KV_HEAD))
    assert call("tsa_select", kvd, sc, idx, None, 0, None) == 6
    assert call("tsa_select", kvd, sc, idx, ws, 8 * 8192 * 4, None) == 6
    assert call("tsa_select", kvd, sc, idx, sc + 4096, big, None) == 7
    # drift
    assert call("tsa_drift", bd, q, None, o, ws, big, None) == 1
    assert call("tsa_drift", bd, q, r, o, None, 0, None) == 6
    assert call("tsa_drift", bd, q, r, o + 4, ws, big, None) == 5
    assert call("tsa_drift", bd, q, r, q + 64, ws, big, None) == 7
    assert call("tsa_drift", bd, q, r, o, r + 4096, big, None) == 7
    assert call("tsa_drift", ctypes.byref(D(keep=2)), q, r, o, ws, 16, None) == 6   # budget not checked
    assert call("tsa_drift", ctypes.byref(D(d=96)), q, r, o, ws, big, None) == 2
    # sparse attention on given subsets
    sa = "tsa_sparse_attn"
    assert call(sa, bd, q, k, v, None, r, o, ws, big, None) == 1
    assert call(sa, bd, q, k, v, idx, r, o, None, 0, None) == 6
    assert call(sa, bd, q, k, v, idx, r, o, ws, 16, None) == 6
    assert call(sa, bd, q, k, v, idx + 4, r, o, ws, big, None) == 5
    assert call(sa, bd, q, k, v, idx, r, q, ws, big, None) == 7            # out over q
    assert call(sa, bd, q, k, v, idx, r, r + 256, ws, big, None) == 7      # partial overlap with the residual
    assert call(sa, bd, q, k, v, idx, r, o, idx + 64, big, None) == 7      # workspace over idx
    assert call(sa, ctypes.byref(D(keep=2)), q, k, v, idx, r, o, ws, big, None) == 3
    # no workspace argument: scores and idx are required, and a problem whose workspace
    # exceeds the static scratch array is rejected before anything runs
    na = "tsa_forward_noalloc"
    assert call(na, bd, q, k, v, r, o, None, idx, None) == 1
    assert call(na, bd, q, k, v, r, o, sc, None, None) == 1
    assert call(na, bd, q, k, v, r, o, sc + 4, idx, None) == 5
    assert call(na, ctypes.byref(D(keep=2)), q, k, v, r, o, sc, idx, None) == 3
    assert call(na, ctypes.byref(D(L=262144, keep=4096)), q, k, v, r, o, sc, idx, None) == 6   # inverse map 33.5 MB
    assert call(na, ctypes.byref(D(L=0, keep=0)), None, None, None, None, None, None, None, None) == 0
    # plain copy
    assert call("tsa_stream_copy", o, None, 4096, None) == 1
    assert call("tsa_stream_copy", o, q, 4095, None) == 5
    assert call("tsa_stream_copy", o + 8, q, 4096, None) == 5
    assert call("tsa_stream_copy", q + 2048, q, 4096, None) == 7
    assert call("tsa_stream_copy", None, None, 0, None) == 0               # nothing to copy
    # descriptor errors come first
    bad = ctypes.byref(D(keep=2))
    assert call("tsa_forward", bad, q, k, v, r, o, None, None, ws, big, None) == 3
    assert call("tsa_dense_attn", ctypes.byref(D(d=32)), q, k, v, o, None) == 2
    assert call("tsa_dense_attn", ctypes.byref(D(keep=2)), None, None, None, None, None) == 1   # keep ignored
    assert call("tsa_forward", None, q, k, v, r, o, None, None, ws, big, None) == 1
