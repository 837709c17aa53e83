"""The C-ABI library: it loads, exports every declared entry point, and rejects
bad arguments on the host before any GPU work (CPU only: every call below fails
validation, so nothing is launched)."""

import ctypes
import subprocess

import pytest

from io_aware_exact_attention_amd import fa355

A = 0x10000        # a 16-byte-aligned fake device address (never dereferenced)
MIS = 0x10008      # 8-byte aligned only


def _fwd(q=A, k=A, v=A, o=A, lse=A, B=1, H=1, Nq=16, Nk=16, d=64, scale=0.125, causal=0):
    return fa355.lib().fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, None)


def _bwd(ptrs=None, ws=A, wsb=1 << 20, B=1, H=1, Nq=16, Nk=16, d=64, scale=0.125, causal=0):
    p = ptrs or [A] * 9
    return fa355.lib().fa_bwd(*p, ws, wsb, B, H, Nq, Nk, d, scale, causal, None)


def _fwd_varlen(cu=A, nseq=2, mq=16, mk=16, H=1, d=64, scale=0.125, causal=0, o=A):
    return fa355.lib().fa_fwd_varlen(A, A, A, o, A, cu, cu, nseq, mq, mk, H, d, scale, causal, None)


def test_exports_every_declared_function():
    names = fa355.header_functions()
    assert set(names) >= {"fa_fwd", "fa_bwd", "fa_fwd_varlen", "fa_bwd_varlen",
                          "fa_bwd_workspace_bytes", "fa_status_string", "fa_version"}
    out = subprocess.run(["nm", "-D", "--defined-only", fa355.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in exported, f"{n} declared in fa355.h but not exported"
        assert hasattr(fa355.lib(), n)


def test_status_strings_and_version():
    for code, name in fa355.STATUS.items():
        assert fa355.fa_status_string(code).startswith(name)
    assert fa355.fa_status_string(-99) == "FA_ERR_UNKNOWN"
    assert fa355.lib().fa_version() >= 100


def test_workspace_bytes():
    assert fa355.fa_bwd_workspace_bytes(8, 16, 4096, 128) == 2 * 4 * 8 * 16 * 4096
    assert fa355.fa_bwd_workspace_bytes(0, 16, 4096, 128) == 0
    assert fa355.fa_bwd_workspace_bytes(2, -1, 4, 64) == 0


@pytest.mark.parametrize("arg", ["q", "k", "v", "o", "lse"])
def test_fwd_null(arg):
    assert _fwd(**{arg: None}) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -2), (dict(H=0), -2), (dict(Nq=0), -2), (dict(Nk=-3), -2),
    (dict(d=96), -3), (dict(d=256), -3), (dict(d=32), -3),
    (dict(causal=1, Nq=16, Nk=32), -3), (dict(causal=2), -3),
    (dict(scale=0.0), -3), (dict(scale=float("nan")), -3), (dict(scale=float("inf")), -3),
    (dict(q=MIS), -4), (dict(o=MIS), -4), (dict(lse=A + 2), -4),
    (dict(B=1 << 20, Nq=1 << 20, Nk=1 << 20), -2),
    # one sequence's key rows of one tensor span 4 GiB: beyond a buffer range
    (dict(H=16, Nq=1 << 20, Nk=1 << 20, d=128), -3),
])
def test_fwd_rejects(kw, code):
    assert _fwd(**kw) == code


def test_bwd_rejects():
    assert _bwd(ptrs=[A] * 8 + [None]) == -1
    assert _bwd(ws=None) == -6
    assert _bwd(wsb=2 * 4 * 16 - 1) == -6
    assert _bwd(d=80) == -3
    assert _bwd(causal=1, Nk=8) == -3
    assert _bwd(ptrs=[A] * 6 + [MIS] + [A] * 2) == -4
    assert _bwd(ws=A + 2) == -4
    assert _bwd(Nq=0) == -2
    assert _bwd(H=16, Nq=1 << 20, Nk=1 << 20, d=128, wsb=1 << 40) == -3


def test_varlen_rejects():
    assert _fwd_varlen(cu=None) == -1
    assert _fwd_varlen(nseq=0) == -2
    assert _fwd_varlen(mq=0) == -2
    assert _fwd_varlen(d=48) == -3
    assert _fwd_varlen(cu=A + 2) == -4
    assert _fwd_varlen(o=MIS) == -4
    lib = fa355.lib()
    assert lib.fa_bwd_varlen(*[A] * 9, A, 4, A, A, 2, 16, 16, 1, 64, 0.1, 0, None) == -6
    assert lib.fa_bwd_varlen(*[A] * 9, A, 1 << 20, None, A, 2, 16, 16, 1, 64, 0.1, 0, None) == -1


def test_stage_entry_points_reject():
    lib = fa355.lib()
    W = 1 << 20
    assert lib.fa_bwd_dot(None, A, A, A, W, 1, 1, 16, 64, None) == -1
    assert lib.fa_bwd_dot(A, A, None, A, W, 1, 1, 16, 64, None) == -1
    assert lib.fa_bwd_dot(A, A, A, A, W, 1, 1, 16, 72, None) == -3
    assert lib.fa_bwd_dot(A, MIS, A, A, W, 1, 1, 16, 64, None) == -4
    assert lib.fa_bwd_dot(A, A, A, None, W, 1, 1, 16, 64, None) == -6
    assert lib.fa_bwd_dot(A, A, A, A, 2 * 4 * 16 - 1, 1, 1, 16, 64, None) == -6
    assert lib.fa_bwd_dkdv(*[A] * 4, A, W, None, A, 1, 1, 16, 16, 64, 0.1, 0, None) == -1
    assert lib.fa_bwd_dkdv(*[A] * 4, A, W, A, A, 1, 1, 16, 8, 64, 0.1, 1, None) == -3
    assert lib.fa_bwd_dkdv(*[A] * 4, A, 8, A, A, 1, 1, 16, 16, 64, 0.1, 0, None) == -6
    assert lib.fa_bwd_dq(*[A] * 4, A, W, None, 1, 1, 16, 16, 64, 0.1, 0, None) == -1
    assert lib.fa_bwd_dq(*[A] * 4, A, W, MIS, 1, 1, 16, 16, 64, 0.1, 0, None) == -4
    assert lib.fa_bwd_dq(*[A] * 4, A, W, A, 1, 1, 0, 16, 64, 0.1, 0, None) == -2

    def dqdot(q=A, o=A, lse=A, ws=A, wsb=W, dq=A, B=1, H=1, Nq=16, Nk=16, d=64, scale=0.1, causal=0):
        return lib.fa_bwd_dq_dot(q, A, A, o, A, lse, ws, wsb, dq, B, H, Nq, Nk, d, scale, causal, None)

    assert dqdot(q=None) == -1 and dqdot(o=None) == -1 and dqdot(lse=None) == -1 and dqdot(dq=None) == -1
    assert dqdot(Nq=0) == -2 and dqdot(B=0) == -2
    assert dqdot(d=72) == -3 and dqdot(Nk=8, causal=1) == -3 and dqdot(scale=0.0) == -3
    assert dqdot(dq=MIS) == -4 and dqdot(o=MIS) == -4
    assert dqdot(ws=None) == -6 and dqdot(wsb=2 * 4 * 16 - 1) == -6


def test_decode_rejects():
    lib = fa355.lib()
    W = 1 << 30

    def dec(q=A, k=A, v=A, o=A, lse=A, ws=A, wsb=W, B=1, Hq=8, Hkv=2, Nq=4, Nk=100, d=128,
            scale=0.1, causal=1):
        return lib.fa_fwd_decode(q, k, v, o, lse, ws, wsb, B, Hq, Hkv, Nq, Nk, d, scale, causal, None)

    assert dec(q=None) == -1 and dec(lse=None) == -1
    assert dec(B=0) == -2 and dec(Nq=0) == -2 and dec(Nk=0) == -2 and dec(Hkv=0) == -2
    assert dec(Hq=6, Hkv=4) == -2                       # Hkv must divide Hq
    assert dec(d=96) == -3 and dec(scale=0.0) == -3
    assert dec(Nq=8, Nk=4, causal=1) == -3              # causal needs Nq <= Nk
    assert dec(Nq=8, Nk=4, causal=0, ws=None) == -6     # non-causal is fine, workspace is not
    assert dec(ws=None) == -6 and dec(wsb=16) == -6
    assert dec(k=MIS) == -4 and dec(ws=A + 4) == -4
    assert dec(Hkv=64, Hq=64, Nk=1 << 17) == -3         # one sequence's cache rows span 2 GiB


def test_decode_workspace_bytes():
    n = fa355.fa_decode_workspace_bytes(2, 32, 4, 4, 131072, 128)
    # two planes of slots (B * Hkv * 32 rows * splits): outputs (d floats) and LSEs
    assert n > 0 and n % (4 * 129) == 0
    assert fa355.fa_decode_workspace_bytes(2, 30, 4, 4, 100, 128) == 0
    assert fa355.fa_decode_workspace_bytes(0, 32, 4, 4, 100, 128) == 0


def test_fp8_rejects():
    lib = fa355.lib()
    W = 1 << 30

    def f8(q=A, k=A, v=A, sg=A, o=A, lse=A, ws=A, wsb=W, B=1, Nq=64, Nk=64, H=2, d=128,
           scale=0.1, causal=1, rotate=1):
        return lib.fa_fwd_fp8(q, k, v, sg, o, lse, ws, wsb, B, Nq, Nk, H, d, scale, causal, rotate, None)

    assert f8(q=None) == -1 and f8(lse=None) == -1
    assert f8(sg=None) == -1                            # rotation needs the signs
    assert f8(sg=None, rotate=0, ws=None) == -6         # ... unless there is none
    assert f8(B=0) == -2 and f8(Nq=0) == -2 and f8(H=0) == -2
    assert f8(d=64) == -3 and f8(scale=float("nan")) == -3 and f8(rotate=2) == -3
    assert f8(Nq=32, Nk=64, causal=1) == -3
    assert f8(ws=None) == -6 and f8(wsb=16) == -6
    assert f8(k=MIS) == -4 and f8(ws=A + 16) == -4 and f8(sg=A + 2) == -4
    assert f8(H=64, Nk=1 << 18) == -3                   # one sequence's code rows span 2 GiB

    def codes(q8=A, k8=A, v8=A, sq=A, sk=A, sv=A, o=A, lse=A, B=1, Nq=64, Nk=64, H=2, d=128,
              qk=0.1, causal=0):
        return lib.fa_fwd_fp8_codes(q8, k8, v8, sq, sk, sv, o, lse, B, Nq, Nk, H, d, qk, causal, None)

    assert codes(sv=None) == -1 and codes(q8=None) == -1
    assert codes(d=64) == -3 and codes(Nq=0) == -2 and codes(qk=-1.0) == -3
    assert codes(o=MIS) == -4 and codes(sk=A + 2) == -4


def test_fp8_workspace_bytes():
    n = fa355.fa_fp8_workspace_bytes(8, 4096, 4096, 16, 128)
    codes = 3 * 8 * 4096 * 16 * 128
    assert codes < n < codes + (1 << 20) and n % 256 == 0
    assert fa355.fa_fp8_workspace_bytes(8, 4096, 4096, 16, 64) == 0
    assert fa355.fa_fp8_workspace_bytes(0, 4096, 4096, 16, 128) == 0


def test_binding_raises_on_error():
    with pytest.raises(fa355.FaError) as e:
        fa355._check(-3)
    assert e.value.status == -3


def test_noalloc_limit_matches_header_and_rejects_larger_calls():
    import re
    text = open(fa355.HEADER).read()
    m = re.search(r"#define FA_BWD_NOALLOC_MAX_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa355.FA_BWD_NOALLOC_MAX_BYTES
    n_rows = fa355.FA_BWD_NOALLOC_MAX_BYTES // 8 + 1   # 8 workspace bytes per (batch, head, row)
    f = fa355.lib().fa_bwd_noalloc
    assert f(*[A] * 9, 1, 1, n_rows, n_rows, 64, 0.125, 0, None) == -6   # FA_ERR_WORKSPACE
    assert f(*[A] * 8, None, 1, 1, 16, 16, 64, 0.125, 0, None) == -1     # FA_ERR_NULL
    assert f(*[A] * 9, 1, 1, 16, 8, 64, 0.125, 1, None) == -3            # causal, Nq != Nk
    assert f(*[A] * 8, MIS, 1, 1, 16, 16, 64, 0.125, 0, None) == -4      # misaligned dv
