"""The binding rejects mismatched buffers with ValueError before calling into the library:
shapes, dtypes, layouts and devices of every tensor an entry point or helper receives are
checked against one another and against the descriptor.  CPU tensors suffice: the shape,
dtype and layout checks come before the device check, and nothing reaches a kernel."""
import pytest
import torch

from tests._lib import ensure_built

tsa = ensure_built()

B, L, H, Hkv, d, keep = 1, 256, 4, 2, 64, 128
bf = torch.bfloat16


def qkvr(dtype=bf):
    q = torch.zeros(B, L, H, d, dtype=dtype)
    k = torch.zeros(B, L, Hkv, d, dtype=dtype)
    v = torch.zeros(B, L, Hkv, d, dtype=dtype)
    r = torch.zeros(B, L, H, d, dtype=dtype)
    return q, k, v, r


def test_forward_checks_every_tensor():
    q, k, v, r = qkvr()
    with pytest.raises(ValueError, match="v must have the shape of k"):
        tsa.forward(q, k, v[:, :, :1].contiguous(), r, keep)
    with pytest.raises(ValueError, match="residual must have the shape of q"):
        tsa.forward(q, k, v, r[:, : L - 1].contiguous(), keep)
    with pytest.raises(ValueError, match="residual must have the dtype of q"):
        tsa.forward(q, k, v, r.float(), keep)
    with pytest.raises(ValueError, match="out must have the shape of residual"):
        tsa.forward(q, k, v, r, keep, out=torch.zeros(B, L, H, d // 2, dtype=bf))
    with pytest.raises(ValueError, match="out must have the dtype"):
        tsa.forward(q, k, v, r, keep, out=torch.zeros(B, L, H, d, dtype=torch.float32))
    with pytest.raises(ValueError, match="contiguous"):
        tsa.forward(q, k, v, r.transpose(1, 2).contiguous().transpose(1, 2), keep)
    with pytest.raises(ValueError, match="k must have the dtype of q"):
        tsa.forward(q, k.float(), v.float(), r, keep)
    with pytest.raises(ValueError, match="H % Hkv"):
        tsa.forward(q, torch.zeros(B, L, 3, d, dtype=bf), torch.zeros(B, L, 3, d, dtype=bf), r, keep)
    with pytest.raises(ValueError, match="ws must"):
        tsa.forward(q, k, v, r, keep, ws=torch.zeros(16, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU device"):          # everything consistent, but on the host
        tsa.forward(q, k, v, r, keep)


def test_helpers_check_index_lists_and_compact_tensors():
    q, k, v, r = qkvr()
    idx = torch.zeros(B, H, keep, dtype=torch.int32)
    with pytest.raises(ValueError, match="idx"):
        tsa.gather_qkv(q, k, v, idx.long())                      # int64 would be read as int32 pairs
    with pytest.raises(ValueError, match="idx must be int32"):
        tsa.gather_qkv(q, k, v, torch.zeros(B, 3, keep, dtype=torch.int32))
    oh = torch.zeros(B, H, keep, d, dtype=bf)
    with pytest.raises(ValueError, match="oh must be"):
        tsa.scatter_residual(oh[:, :, :-1].contiguous(), idx, r)
    with pytest.raises(ValueError, match="oh must be"):
        tsa.scatter_residual(oh.float(), idx, r)
    with pytest.raises(ValueError, match="out must have the shape"):
        tsa.scatter_residual(oh, idx, r, out=torch.zeros(B, L - 1, H, d, dtype=bf))
    with pytest.raises(ValueError, match="idx must be int32"):         # 3 subset rows cannot serve 4 heads
        tsa.scatter_residual(oh, torch.zeros(B, 3, keep, dtype=torch.int32), r)
    with pytest.raises(ValueError, match="GPU device"):                # one row per KV head (R = 2) is fine
        tsa.scatter_residual(oh, torch.zeros(B, Hkv, keep, dtype=torch.int32), r)
    with pytest.raises(ValueError, match="kh, vh"):
        tsa.attn(oh, torch.zeros(B, 3, keep, d, dtype=bf), torch.zeros(B, 3, keep, d, dtype=bf))
    with pytest.raises(ValueError, match="vh must have the shape of kh"):
        tsa.attn(oh, oh, oh[:, :2].contiguous())
    with pytest.raises(ValueError, match="idx"):
        tsa.sparse_attn(q, k, v, idx.long(), r)
    with pytest.raises(ValueError, match="scores"):
        tsa.select(torch.zeros(B, H, L, dtype=torch.float64), keep)
    with pytest.raises(ValueError, match="kv_heads"):
        tsa.select(torch.zeros(B, H, L), keep, kv_heads=3)
    with pytest.raises(ValueError, match="h_after must have the shape"):
        tsa.drift(r, r[:, :-1].contiguous())
    with pytest.raises(ValueError, match="GPU device"):
        tsa.gather_qkv(q, k, v, idx)


def test_raw_entry_points_check_buffers_against_the_descriptor():
    q, k, v, r = qkvr()
    desc = tsa.desc_for(q, k, keep, W=32, n_sink=4)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    with pytest.raises(ValueError, match="out holds"):           # too small: would be written out of bounds
        tsa.tsa_forward(desc, q, k, v, r, torch.zeros(B, L // 2, H, d, dtype=bf), None, None, ws)
    with pytest.raises(ValueError, match="residual must be"):
        tsa.tsa_forward(desc, q, k, v, r.float(), r, None, None, ws)
    with pytest.raises(ValueError, match="idx must be torch.int32"):
        tsa.tsa_gather_qkv(desc, q, k, v, torch.zeros(B, H, keep, dtype=torch.int64), q, k, v)
    with pytest.raises(ValueError, match="exceeds"):
        tsa.tsa_forward(desc, q, k, v, r, r, None, None, ws, ws_bytes=(1 << 20) + 1)
    with pytest.raises(ValueError, match="scores must be torch.float32"):
        tsa.tsa_score(desc, q, k, torch.zeros(B, H, L, dtype=torch.float64), ws)
    with pytest.raises(ValueError, match="holds fewer"):
        tsa.tsa_stream_copy(torch.zeros(16, dtype=torch.uint8), torch.zeros(32, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU device"):
        tsa.tsa_forward(desc, q, k, v, r, r.clone(), None, None, ws)
