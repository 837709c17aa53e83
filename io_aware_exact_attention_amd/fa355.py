"""Python binding of libfa355 (ctypes).  Argument marshalling only.

The functions named like the C entry points (``fa_fwd``, ``fa_fwd_persistent``,
``fa_bwd`` and its stages ``fa_bwd_dq_dot`` / ``fa_bwd_dot`` / ``fa_bwd_dkdv`` /
``fa_bwd_dq``, ``fa_bwd_noalloc`` (the backward without a caller workspace),
``fa_fwd_varlen``, ``fa_bwd_varlen``, ``fa_fwd_decode``, ``fa_fwd_fp8``,
``fa_fwd_fp8_codes``, the ``*_workspace_bytes`` queries, ``fa_status_string``)
take torch tensors that already live on the GPU, pass their device pointers and
sizes to the library on the current torch stream, and raise ``FaError`` on a
non-zero status.  Every computation happens in the library's HIP kernels; there
is no other code path, and a missing or unloadable library raises immediately.

``attention_forward`` / ``attention_backward`` (and the varlen, decoding and
FP8 variants) are conveniences that allocate the outputs (and workspaces) with
torch and call the entry points.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa355.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fa355.h")

_c_int, _c_float, _vp, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

_SIGNATURES = {
    "fa_status_string": (ctypes.c_char_p, [_c_int]),
    "fa_version": (_c_int, []),
    "fa_fwd": (_c_int, [_vp] * 5 + [_c_int] * 5 + [_c_float, _c_int, _vp]),
    "fa_fwd_persistent": (_c_int, [_vp] * 5 + [_c_int] * 5 + [_c_float, _c_int, _vp]),
    "fa_fwd_varlen": (_c_int, [_vp] * 7 + [_c_int] * 5 + [_c_float, _c_int, _vp]),
    "fa_bwd_workspace_bytes": (_sz, [_c_int] * 4),
    "fa_bwd": (_c_int, [_vp] * 10 + [_sz] + [_c_int] * 5 + [_c_float, _c_int, _vp]),
    "fa_bwd_noalloc": (_c_int, [_vp] * 9 + [_c_int] * 5 + [_c_float, _c_int, _vp]),
    "fa_bwd_varlen": (_c_int, [_vp] * 10 + [_sz] + [_vp] * 2 + [_c_int] * 5 + [_c_float, _c_int, _vp]),
    "fa_bwd_dot": (_c_int, [_vp] * 4 + [_sz] + [_c_int] * 4 + [_vp]),
    "fa_bwd_dkdv": (_c_int, [_vp] * 5 + [_sz] + [_vp] * 2 + [_c_int] * 5 + [_c_float, _c_int, _vp]),
    "fa_bwd_dq": (_c_int, [_vp] * 5 + [_sz] + [_vp] + [_c_int] * 5 + [_c_float, _c_int, _vp]),
    "fa_bwd_dq_dot": (_c_int, [_vp] * 7 + [_sz] + [_vp] + [_c_int] * 5 + [_c_float, _c_int, _vp]),
    "fa_decode_workspace_bytes": (_sz, [_c_int] * 6),
    "fa_fwd_decode": (_c_int, [_vp] * 6 + [_sz] + [_c_int] * 6 + [_c_float, _c_int, _vp]),
    "fa_fp8_workspace_bytes": (_sz, [_c_int] * 5),
    "fa_fwd_fp8": (_c_int, [_vp] * 7 + [_sz] + [_c_int] * 5 + [_c_float, _c_int, _c_int, _vp]),
    "fa_fwd_fp8_codes": (_c_int, [_vp] * 8 + [_c_int] * 5 + [_c_float, _c_int, _vp]),
}

STATUS = {0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_SHAPE", -3: "FA_ERR_UNSUPPORTED",
          -4: "FA_ERR_ALIGN", -5: "FA_ERR_LAUNCH", -6: "FA_ERR_WORKSPACE"}

# bytes of fa_bwd_noalloc's static device array (FA_BWD_NOALLOC_MAX_BYTES in fa355.h)
FA_BWD_NOALLOC_MAX_BYTES = 16 << 20

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libfa355 error {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m io_aware_exact_attention_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/fa355.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(fa_[a-z0-9_]+)\s*\(", text, re.M)))


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise FaError(status, fa_status_string(status))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_BF16, _F32, _U8, _I32 = torch.bfloat16, torch.float32, torch.uint8, torch.int32


class _Args:
    """Checks of the tensors one call passes: what the C ABI cannot see through
    a bare pointer -- the element type, a non-contiguous layout, a shape that
    disagrees with the sizes passed -- and, once all of those hold, that every
    tensor is in the memory of one GPU."""

    def __init__(self):
        self.seen = []

    def need(self, name, t, dtype=None, shape=None, numel=None):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if numel is not None and t.numel() != int(numel):
            raise ValueError(f"{name} has {t.numel()} elements, expected {int(numel)}")
        self.seen.append((name, t))
        return self

    def on_gpu(self):
        dev = None
        for name, t in self.seen:
            if t.device.type != "cuda":
                raise ValueError(f"{name} must be in GPU memory, got {t.device}")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dense_dims(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("dense tensors are [B, N, H, d]")
    B, Nq, H, d = q.shape
    return B, H, Nq, k.shape[1], d


def _check_dense(q, k, v, o=None, lse=None, extra=(), more=()):
    """q [B,Nq,H,d], k and v [B,Nk,H,d] bf16, o like q, lse [B,H,Nq] fp32;
    extra: (name, tensor, like) with like 'q' or 'k' for more bf16 tensors;
    more: (name, tensor, dtype, shape) checked as given (shape None: any)."""
    B, H, Nq, Nk, d = _dense_dims(q, k)
    a = _Args().need("q", q, _BF16)
    a.need("k", k, _BF16, (B, Nk, H, d)).need("v", v, _BF16, (B, Nk, H, d))
    if o is not None:
        a.need("o", o, _BF16, (B, Nq, H, d))
    if lse is not None:
        a.need("lse", lse, _F32, (B, H, Nq))
    for name, t, like in extra:
        a.need(name, t, _BF16, (B, Nq, H, d) if like == "q" else (B, Nk, H, d))
    for name, t, dtype, shape in more:
        a.need(name, t, dtype, shape)
    a.on_gpu()
    return B, H, Nq, Nk, d


def fa_fwd(q, k, v, o, lse, scale: float, causal: bool, stream=None):
    B, H, Nq, Nk, d = _check_dense(q, k, v, o, lse)
    _check(lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                        float(scale), int(bool(causal)), _stream(stream)))


def fa_fwd_persistent(q, k, v, o, lse, scale: float, causal: bool, stream=None):
    B, H, Nq, Nk, d = _check_dense(q, k, v, o, lse)
    _check(lib().fa_fwd_persistent(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                                   float(scale), int(bool(causal)), _stream(stream)))


def fa_bwd_workspace_bytes(batch_or_nseq: int, H: int, nq: int, d: int) -> int:
    return int(lib().fa_bwd_workspace_bytes(int(batch_or_nseq), int(H), int(nq), int(d)))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, scale: float, causal: bool, stream=None):
    B, H, Nq, Nk, d = _check_dense(q, k, v, o, lse,
                                   (("dout", dout, "q"), ("dq", dq, "q"), ("dk", dk, "k"), ("dv", dv, "k")),
                                   (("workspace", workspace, None, None),))
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                        _ptr(dk), _ptr(dv), _ptr(workspace), nbytes, B, H, Nq, Nk, d,
                        float(scale), int(bool(causal)), _stream(stream)))


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, scale: float, causal: bool, stream=None):
    B, H, Nq, Nk, d = _check_dense(q, k, v, o, lse,
                                   (("dout", dout, "q"), ("dq", dq, "q"), ("dk", dk, "k"), ("dv", dv, "k")))
    _check(lib().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                _ptr(dk), _ptr(dv), B, H, Nq, Nk, d, float(scale), int(bool(causal)),
                                _stream(stream)))


def fa_bwd_dq_dot(q, k, v, o, dout, lse, workspace, dq, scale: float, causal: bool, stream=None):
    B, H, Nq, Nk, d = _check_dense(q, k, v, o, lse, extra=(("dout", dout, "q"), ("dq", dq, "q")),
                                   more=(("workspace", workspace, None, None),))
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fa_bwd_dq_dot(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                               _ptr(workspace), nbytes, _ptr(dq), B, H, Nq, Nk, d, float(scale),
                               int(bool(causal)), _stream(stream)))


def fa_bwd_dot(o, dout, lse, workspace, stream=None):
    if o.dim() != 4:
        raise ValueError("dense tensors are [B, N, H, d]")
    B, Nq, H, d = o.shape
    (_Args().need("o", o, _BF16).need("dout", dout, _BF16, o.shape).need("lse", lse, _F32, (B, H, Nq))
     .need("workspace", workspace).on_gpu())
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fa_bwd_dot(_ptr(o), _ptr(dout), _ptr(lse), _ptr(workspace), nbytes, B, H, Nq, d,
                            _stream(stream)))


def fa_bwd_dkdv(q, k, v, dout, workspace, dk, dv, scale: float, causal: bool, stream=None):
    B, H, Nq, Nk, d = _check_dense(q, k, v, extra=(("dout", dout, "q"), ("dk", dk, "k"), ("dv", dv, "k")),
                                   more=(("workspace", workspace, None, None),))
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(workspace), nbytes,
                             _ptr(dk), _ptr(dv), B, H, Nq, Nk, d, float(scale),
                             int(bool(causal)), _stream(stream)))


def fa_bwd_dq(q, k, v, dout, workspace, dq, scale: float, causal: bool, stream=None):
    B, H, Nq, Nk, d = _check_dense(q, k, v, extra=(("dout", dout, "q"), ("dq", dq, "q")),
                                   more=(("workspace", workspace, None, None),))
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(workspace), nbytes,
                           _ptr(dq), B, H, Nq, Nk, d, float(scale), int(bool(causal)),
                           _stream(stream)))


def _check_packed(q, k, v, o, lse, cu_q, cu_k, max_q, extra=(), more=()):
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("packed tensors are [total, H, d]")
    a = _Args().need("q", q, _BF16).need("cu_seqlens_q", cu_q, _I32)
    nseq = cu_q.numel() - 1
    a.need("cu_seqlens_k", cu_k, _I32, (nseq + 1,)).need("k", k, _BF16).need("v", v, _BF16, k.shape)
    a.need("o", o, _BF16, q.shape).need("lse", lse, _F32, (nseq, q.shape[1], int(max_q)))
    for name, t, like in extra:
        a.need(name, t, _BF16, q.shape if like == "q" else k.shape)
    for name, t, dtype, shape in more:
        a.need(name, t, dtype, shape)
    a.on_gpu()
    return nseq


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                  max_seqlen_k: int, scale: float, causal: bool, stream=None):
    nseq = _check_packed(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q)
    _check(lib().fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens_q),
                               _ptr(cu_seqlens_k), nseq, int(max_seqlen_q), int(max_seqlen_k),
                               q.shape[1], q.shape[2], float(scale), int(bool(causal)),
                               _stream(stream)))


def fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, workspace, cu_seqlens_q, cu_seqlens_k,
                  max_seqlen_q: int, max_seqlen_k: int, scale: float, causal: bool, stream=None):
    nseq = _check_packed(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                         (("dout", dout, "q"), ("dq", dq, "q"), ("dk", dk, "k"), ("dv", dv, "k")),
                         (("workspace", workspace, None, None),))
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fa_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                               _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), nbytes,
                               _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), nseq, int(max_seqlen_q),
                               int(max_seqlen_k), q.shape[1], q.shape[2], float(scale),
                               int(bool(causal)), _stream(stream)))


def fa_decode_workspace_bytes(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int) -> int:
    return int(lib().fa_decode_workspace_bytes(int(B), int(Hq), int(Hkv), int(Nq), int(Nk), int(d)))


def fa_fwd_decode(q, k, v, o, lse, workspace, scale: float, causal: bool, stream=None):
    """q [B,Nq,Hq,d]; k, v [B,Nk,Hkv,d]; o like q; lse [B,Hq,Nq] fp32."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q [B,Nq,Hq,d]; k, v [B,Nk,Hkv,d]")
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    (_Args().need("q", q, _BF16).need("k", k, _BF16, (B, Nk, Hkv, d)).need("v", v, _BF16, (B, Nk, Hkv, d))
     .need("o", o, _BF16, q.shape).need("lse", lse, _F32, (B, Hq, Nq)).need("workspace", workspace)
     .on_gpu())
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fa_fwd_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
                               nbytes, B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                               _stream(stream)))


def fa_fp8_workspace_bytes(B: int, Nq: int, Nk: int, H: int, d: int) -> int:
    return int(lib().fa_fp8_workspace_bytes(B, Nq, Nk, H, d))


def fa_fwd_fp8(q, k, v, signs, o, lse, workspace, scale: float, causal: bool, rotate: bool = True,
               stream=None):
    """q [B,Nq,H,d]; k, v [B,Nk,H,d] bf16; signs fp32 [d]; o like q; lse [B,H,Nq] fp32."""
    more = [("workspace", workspace, None, None)]
    if rotate or signs is not None:
        more.append(("signs", signs, _F32, (q.shape[-1],)))
    B, H, Nq, Nk, d = _check_dense(q, k, v, o, lse, more=more)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(signs),
                            _ptr(o), _ptr(lse), _ptr(workspace), nbytes, B, Nq, Nk, H, d,
                            float(scale), int(bool(causal)), int(bool(rotate)), _stream(stream)))


def fa_fwd_fp8_codes(q8, k8, v8, sq, sk, sv, o, lse, qk_scale: float, causal: bool, stream=None):
    """q8 [B,Nq,H,d], k8, v8 [B,Nk,H,d] uint8 e4m3 codes; sq [B*H*ceil(Nq/64)], sk, sv
    [B*H*ceil(Nk/64)] fp32 power-of-two scales, one per 64-row block."""
    if q8.dim() != 4 or k8.dim() != 4:
        raise ValueError("codes are [B, N, H, d]")
    B, Nq, H, d = q8.shape
    Nk = k8.shape[1]
    (_Args().need("q8", q8, _U8).need("k8", k8, _U8, (B, Nk, H, d)).need("v8", v8, _U8, (B, Nk, H, d))
     .need("sq", sq, _F32, numel=B * H * ((Nq + 63) // 64))
     .need("sk", sk, _F32, numel=B * H * ((Nk + 63) // 64))
     .need("sv", sv, _F32, numel=B * H * ((Nk + 63) // 64))
     .need("o", o, _BF16, (B, Nq, H, d)).need("lse", lse, _F32, (B, H, Nq)).on_gpu())
    _check(lib().fa_fwd_fp8_codes(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(sq), _ptr(sk), _ptr(sv),
                                  _ptr(o), _ptr(lse), B, Nq, Nk, H, d, float(qk_scale),
                                  int(bool(causal)), _stream(stream)))


def fp8_workspace_views(workspace, B: int, Nq: int, Nk: int, H: int, d: int):
    """The codes and scales fa_fwd_fp8 leaves in its workspace (views, no copies).

    Offsets follow the documented layout: q8, k8, v8, then scales [3, B, H, nblk]
    (one per 64-row block, nblk for the longer of q and k), each start rounded up
    to 256 bytes.
    """
    def up(x):
        return (x + 255) // 256 * 256
    w = workspace.view(torch.uint8)
    bh = B * H
    o_k = up(bh * Nq * d)
    o_v = o_k + up(bh * Nk * d)
    o_s = o_v + up(bh * Nk * d)
    q8 = w[:bh * Nq * d].view(B, Nq, H, d)
    k8 = w[o_k:o_k + bh * Nk * d].view(B, Nk, H, d)
    v8 = w[o_v:o_v + bh * Nk * d].view(B, Nk, H, d)
    nblk = (max(Nq, Nk) + 63) // 64
    scales = w[o_s:o_s + 12 * bh * nblk].view(torch.float32).view(3, B, H, nblk)
    return q8, k8, v8, scales


# ---------------------------------------------------------------------------
# conveniences: allocate outputs (device memory via torch), then call the ABI

def attention_forward(q, k, v, scale: float, causal: bool):
    B, H, Nq, Nk, d = _dense_dims(q, k)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, Nq, dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, scale, causal)
    return o, lse


def attention_backward(q, k, v, o, dout, lse, scale: float, causal: bool, workspace=None):
    B, H, Nq, Nk, d = _dense_dims(q, k)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        nbytes = fa_bwd_workspace_bytes(B, H, Nq, d)
        workspace = torch.empty(nbytes // 4, dtype=torch.float32, device=q.device)
    fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, scale, causal)
    return dq, dk, dv


def attention_forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                             scale: float, causal: bool):
    nseq = cu_seqlens_q.numel() - 1
    o = torch.empty_like(q)
    lse = torch.empty(nseq, q.shape[1], max_seqlen_q, dtype=torch.float32, device=q.device)
    fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                  scale, causal)
    return o, lse


def attention_backward_varlen(q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                              max_seqlen_k, scale: float, causal: bool, workspace=None):
    nseq = cu_seqlens_q.numel() - 1
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        nbytes = fa_bwd_workspace_bytes(nseq, q.shape[1], max_seqlen_q, q.shape[2])
        workspace = torch.empty(nbytes // 4, dtype=torch.float32, device=q.device)
    fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, workspace, cu_seqlens_q, cu_seqlens_k,
                  max_seqlen_q, max_seqlen_k, scale, causal)
    return dq, dk, dv


def attention_decode(q, k, v, scale: float, causal: bool, workspace=None):
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, Nq, dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = fa_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, d)
        workspace = torch.empty(max(nbytes, 16) // 4, dtype=torch.float32, device=q.device)
    fa_fwd_decode(q, k, v, o, lse, workspace, scale, causal)
    return o, lse


def attention_forward_fp8(q, k, v, signs, scale: float, causal: bool, rotate: bool = True,
                          workspace=None):
    B, H, Nq, Nk, d = _dense_dims(q, k)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, Nq, dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = fa_fp8_workspace_bytes(B, Nq, Nk, H, d)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    fa_fwd_fp8(q, k, v, signs, o, lse, workspace, scale, causal, rotate)
    return o, lse
