"""The Python binding refuses, before calling the library, what a bare pointer
cannot carry: wrong element types, non-contiguous layouts, shapes that disagree
with the sizes it passes, and tensors outside GPU memory (CPU only)."""

import pytest
import torch

from io_aware_exact_attention_amd import fa355

BF, F32 = torch.bfloat16, torch.float32


def _z(*shape, dtype=BF):
    return torch.zeros(*shape, dtype=dtype)


def _noncontig(*shape, dtype=BF):
    t = torch.zeros(*reversed(shape), dtype=dtype)
    return t.permute(*reversed(range(len(shape))))


def test_dense_forward_checks():
    q, lse = _z(1, 16, 2, 64), _z(1, 2, 16, dtype=F32)
    with pytest.raises(TypeError, match="q must be torch.bfloat16"):
        fa355.fa_fwd(q.float(), q, q, q, lse, 0.1, False)
    with pytest.raises(ValueError, match="k must be contiguous"):
        fa355.fa_fwd(q, _noncontig(1, 16, 2, 64), q, q, lse, 0.1, False)
    with pytest.raises(ValueError, match="v has shape"):
        fa355.fa_fwd(q, q, _z(1, 16, 2, 128), q, lse, 0.1, False)
    with pytest.raises(ValueError, match="lse has shape"):
        fa355.fa_fwd(q, q, q, q, _z(1, 2, 15, dtype=F32), 0.1, False)
    with pytest.raises(TypeError, match="lse must be torch.float32"):
        fa355.fa_fwd_persistent(q, q, q, q, _z(1, 2, 16), 0.1, False)
    with pytest.raises(ValueError, match="in GPU memory"):
        fa355.fa_fwd(q, q, q, q, lse, 0.1, False)
    with pytest.raises(ValueError, match=r"\[B, N, H, d\]"):
        fa355.fa_fwd(q[0], q, q, q, lse, 0.1, False)


def test_backward_checks():
    q, lse, ws = _z(1, 16, 2, 64), _z(1, 2, 16, dtype=F32), _z(256, dtype=F32)
    with pytest.raises(ValueError, match="dk has shape"):
        fa355.fa_bwd(q, q, q, q, q, lse, q, _z(1, 8, 2, 64), q, ws, 0.1, False)
    with pytest.raises(TypeError, match="dout must be"):
        fa355.fa_bwd_dot(q, q.float(), lse, ws)
    with pytest.raises(ValueError, match="workspace must be contiguous"):
        fa355.fa_bwd_dq(q, q, q, q, _noncontig(16, 16, dtype=F32), q, 0.1, False)
    with pytest.raises(ValueError, match="in GPU memory"):
        fa355.fa_bwd_dkdv(q, q, q, q, ws, q, q, 0.1, False)


def test_packed_checks():
    q, cu = _z(40, 2, 64), torch.tensor([0, 10, 40], dtype=torch.int32)
    lse = _z(2, 2, 30, dtype=F32)
    with pytest.raises(TypeError, match="cu_seqlens_q must be torch.int32"):
        fa355.fa_fwd_varlen(q, q, q, q, lse, cu.long(), cu, 30, 30, 0.1, True)
    with pytest.raises(ValueError, match="cu_seqlens_k has shape"):
        fa355.fa_fwd_varlen(q, q, q, q, lse, cu, cu[:2], 30, 30, 0.1, True)
    with pytest.raises(ValueError, match="lse has shape"):
        fa355.fa_fwd_varlen(q, q, q, q, lse, cu, cu, 31, 30, 0.1, True)
    with pytest.raises(ValueError, match="in GPU memory"):
        fa355.fa_bwd_varlen(q, q, q, q, q, lse, q, q, q, _z(64, dtype=F32), cu, cu, 30, 30, 0.1, True)


def test_decode_and_fp8_checks():
    q, k = _z(1, 4, 8, 128), _z(1, 100, 2, 128)
    ws = _z(64, dtype=F32)
    with pytest.raises(ValueError, match="lse has shape"):
        fa355.fa_fwd_decode(q, k, k, q, _z(1, 4, 8, dtype=F32), ws, 0.1, True)
    with pytest.raises(ValueError, match="in GPU memory"):
        fa355.fa_fwd_decode(q, k, k, q, _z(1, 8, 4, dtype=F32), ws, 0.1, True)
    x, lse = _z(1, 64, 2, 128), _z(1, 2, 64, dtype=F32)
    with pytest.raises(ValueError, match="signs has shape"):
        fa355.fa_fwd_fp8(x, x, x, _z(64, dtype=F32), x, lse, _z(8, dtype=torch.uint8), 0.1, True)
    with pytest.raises(ValueError, match="in GPU memory"):
        fa355.fa_fwd_fp8(x, x, x, None, x, lse, _z(8, dtype=torch.uint8), 0.1, True, rotate=False)
    c8 = _z(1, 64, 2, 128, dtype=torch.uint8)
    s1 = _z(2, dtype=F32)
    with pytest.raises(TypeError, match="q8 must be torch.uint8"):
        fa355.fa_fwd_fp8_codes(x, c8, c8, s1, s1, s1, x, lse, 0.1, True)
    with pytest.raises(ValueError, match="sk has 3 elements"):
        fa355.fa_fwd_fp8_codes(c8, c8, c8, s1, _z(3, dtype=F32), s1, x, lse, 0.1, True)
    with pytest.raises(ValueError, match="in GPU memory"):
        fa355.fa_fwd_fp8_codes(c8, c8, c8, s1, s1, s1, x, lse, 0.1, True)
