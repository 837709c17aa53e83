"""Full-size workloads on the GPU, compared with the oracle on every head.

Each workload runs once at its real size through the same entry points and
launch configuration the benchmark times (fa_fwd + fa_bwd, or their varlen
forms), with every output buffer filled with NaN beforehand, so that a tile a
kernel never writes (or writes under the wrong head) cannot pass as a stale
value.  Heads (and packed sequences) are independent, so the oracle computes each
(batch, head) slice exactly from that slice's inputs alone, and every output
element of the slice is compared at the usual tolerances.  The comparison is
split into one test per batch entry, head or group of sequences, all sharing
the one GPU run, so that each test stays short and reports its own slice.

Oracle time on 8 CPU cores: the headline 4.2 s per batch entry (8 entries),
the long context 11.5 s per head (16 heads), the packed batch about 15 s for
every sequence on two heads.

Every head is also checked on properties that hold at any size: all outputs
finite, and under the causal mask query row 0 sees only key 0, so O[0] = V[0]
exactly and LSE[0] = scale * q0.k0.
"""

import pytest
import torch

from io_aware_exact_attention_amd import fa355, workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

HEADLINE = "b8_h16_n4096_d128_causal"
LONG = "b1_h16_n32768_d128_k3_causal"
VARLEN = "varlen_h32_d128_64seq"


def _nan_like(t):
    return torch.full_like(t, float("nan"))


def _run_dense(name):
    gu.need_gpu()
    w = wl.WORKLOADS[name]
    causal = w.causal[-1]
    gu.announce(f"{name} full size on the GPU (NaN-filled outputs)")
    x = wl.make_inputs(name)
    dev = torch.device("cuda", 0)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    B, N, H, d = q.shape
    o = _nan_like(q)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    fa355.fa_fwd(q, k, v, o, lse, w.scale, causal)
    dq, dk, dv = _nan_like(q), _nan_like(k), _nan_like(v)
    ws = torch.full((fa355.fa_bwd_workspace_bytes(B, H, N, d) // 4,), float("nan"),
                    dtype=torch.float32, device=dev)
    fa355.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, w.scale, causal)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t).all()
    if causal:
        assert torch.equal(o[:, 0], v[:, 0])
        s00 = w.scale * (q[:, 0].float() * k[:, 0].float()).sum(-1)      # [B, H]
        assert (lse[:, :, 0] - s00).abs().max().item() <= gu.LSE_TOL
    out = {n: t.cpu() for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
    return w, x, out


@pytest.fixture(scope="module")
def headline():
    return _run_dense(HEADLINE)


@pytest.fixture(scope="module")
def long_context():
    return _run_dense(LONG)


def _compare_slice(w, x, out, b, hs, what):
    """Batch entry b, heads hs (a slice): oracle on those inputs alone."""
    causal = w.causal[-1]
    sl = (slice(b, b + 1), slice(None), hs)
    xs = {n: x[n][sl].contiguous() for n in ("q", "k", "v", "dout")}
    r = gu.oracle_dense(xs, w.scale, causal)
    gu.check_forward(out["o"][sl], out["lse"][b:b + 1, hs], r["o"], r["lse"], what)
    gu.check_grads((out["dq"][sl], out["dk"][sl], out["dv"][sl]), r["grads"], what)


@pytest.mark.parametrize("b", range(8))
def test_headline_every_head(headline, b):
    w, x, out = headline
    gu.announce(f"{HEADLINE}: batch entry {b}, all 16 heads against the oracle")
    _compare_slice(w, x, out, b, slice(None), f"{HEADLINE} b={b}")


@pytest.mark.parametrize("h", range(16))
def test_long_context_every_head(long_context, h):
    w, x, out = long_context
    gu.announce(f"{LONG}: head {h} against the oracle")
    _compare_slice(w, x, out, 0, slice(h, h + 1), f"{LONG} h={h}")


@pytest.fixture(scope="module")
def varlen():
    gu.need_gpu()
    w = wl.WORKLOADS[VARLEN]
    gu.announce(f"{VARLEN} full size on the GPU (NaN-filled outputs)")
    x = wl.make_inputs(w.name)
    dev = torch.device("cuda", 0)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    cu = x["cu_seqlens"].to(dev)
    mx = x["max_seqlen"]
    nseq = cu.numel() - 1
    o = _nan_like(q)
    lse = torch.full((nseq, w.H, mx), float("nan"), dtype=torch.float32, device=dev)
    fa355.fa_fwd_varlen(q, k, v, o, lse, cu, cu, mx, mx, w.scale, True)
    dq, dk, dv = _nan_like(q), _nan_like(k), _nan_like(v)
    ws = torch.full((fa355.fa_bwd_workspace_bytes(nseq, w.H, mx, w.d) // 4,), float("nan"),
                    dtype=torch.float32, device=dev)
    fa355.fa_bwd_varlen(q, k, v, o, do, lse, dq, dk, dv, ws, cu, cu, mx, mx, w.scale, True)
    torch.cuda.synchronize()
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t).all()
    cu_h = x["cu_seqlens"].tolist()
    starts = torch.tensor(cu_h[:-1], device=dev, dtype=torch.long)
    assert torch.equal(o[starts], v[starts])          # row 0 of every sequence
    lse_c = lse.cpu()
    for s in range(nseq):                             # every written LSE row is finite
        assert torch.isfinite(lse_c[s, :, : cu_h[s + 1] - cu_h[s]]).all()
    out = {n: t.cpu() for n, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv))}
    out["lse"] = lse_c
    return w, x, out


@pytest.mark.parametrize("group", range(8))
def test_varlen_every_sequence_two_heads(varlen, group):
    """Sequences 8*group .. 8*group+7, each on heads s % 32 and (s + 16) % 32."""
    w, x, out = varlen
    cu_h = x["cu_seqlens"].tolist()
    for s in range(8 * group, 8 * group + 8):
        a, e = cu_h[s], cu_h[s + 1]
        for h in (s % w.H, (s + w.H // 2) % w.H):
            gu.announce(f"{VARLEN}: sequence {s} (length {e - a}) head {h}")
            xs = {n: x[n][None, a:e, h:h + 1].contiguous() for n in ("q", "k", "v", "dout")}
            r = gu.oracle_dense(xs, w.scale, True)
            what = f"sequence {s} (length {e - a}) head {h}"
            gu.check_forward(out["o"][None, a:e, h:h + 1], out["lse"][s:s + 1, h:h + 1, : e - a],
                             r["o"], r["lse"], what)
            gu.check_grads((out["dq"][None, a:e, h:h + 1], out["dk"][None, a:e, h:h + 1],
                            out["dv"][None, a:e, h:h + 1]), r["grads"], what)
