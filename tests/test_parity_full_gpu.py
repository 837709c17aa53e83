"""Full-size workloads on the GPU, compared with the oracle on sampled slices.

Each workload runs at its real size through the same entry points and launch
configuration the benchmark times.  Heads (and packed sequences) are
independent, so the oracle computes a sampled (batch, head) slice exactly from
that slice's inputs alone; every output element of the slice is compared.
Every head is also checked on properties that hold at any size: all outputs
finite, and under the causal mask query row 0 sees only key 0, so O[0] = V[0]
exactly and LSE[0] = scale * q0.k0.
"""

import pytest
import torch

import oracle
from io_aware_exact_attention_amd import fa355, workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _dense_full(name, samples):
    gu.need_gpu()
    w = wl.WORKLOADS[name]
    causal = w.causal[-1]
    gu.announce(f"{name} full size, samples {samples}")
    x = wl.make_inputs(name)
    dev = torch.device("cuda", 0)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    o, lse = fa355.attention_forward(q, k, v, w.scale, causal)
    dq, dk, dv = fa355.attention_backward(q, k, v, o, do, lse, w.scale, causal)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t).all()
    if causal:
        assert torch.equal(o[:, 0], v[:, 0])
        s00 = w.scale * (q[:, 0].float() * k[:, 0].float()).sum(-1)      # [B, H]
        assert (lse[:, :, 0] - s00).abs().max().item() <= gu.LSE_TOL
    for b, h in samples:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        xs = {n: x[n][sl].contiguous() for n in ("q", "k", "v", "dout")}
        r = gu.oracle_dense(xs, w.scale, causal)
        what = f"{name} b={b} h={h}"
        gu.check_forward(o[sl], lse[b:b + 1, h:h + 1], r["o"], r["lse"], what)
        gu.check_grads((dq[sl], dk[sl], dv[sl]), r["grads"], what)


def test_headline_b8_h16_n4096_d128_causal():
    _dense_full("b8_h16_n4096_d128_causal", [(0, 0), (3, 7), (7, 15)])


def test_long_context_b1_h16_n32768_d128_causal():
    _dense_full("b1_h16_n32768_d128_k3_causal", [(0, 5)])


def test_varlen_64_sequences():
    gu.need_gpu()
    w = wl.WORKLOADS["varlen_h32_d128_64seq"]
    gu.announce(f"{w.name} full size")
    x = wl.make_inputs(w.name)
    lens = x["lengths"]
    dev = torch.device("cuda", 0)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    cu = x["cu_seqlens"].to(dev)
    mx = x["max_seqlen"]
    o, lse = fa355.attention_forward_varlen(q, k, v, cu, cu, mx, mx, w.scale, True)
    dq, dk, dv = fa355.attention_backward_varlen(q, k, v, o, do, lse, cu, cu, mx, mx, w.scale, True)
    torch.cuda.synchronize()
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t).all()
    cu_h = x["cu_seqlens"].tolist()
    starts = torch.tensor(cu_h[:-1], device=dev, dtype=torch.long)
    assert torch.equal(o[starts], v[starts])          # row 0 of every sequence
    longest = max(range(len(lens)), key=lambda i: lens[i])
    shortest = min(range(len(lens)), key=lambda i: lens[i])
    for s, h in ((longest, 3), (shortest, 30), (17, 0)):
        a, e = cu_h[s], cu_h[s + 1]
        xs = {n: x[n][None, a:e, h:h + 1].contiguous() for n in ("q", "k", "v", "dout")}
        r = gu.oracle_dense(xs, w.scale, True)
        what = f"sequence {s} (length {e - a}) head {h}"
        gu.check_forward(o[None, a:e, h:h + 1], lse[s:s + 1, h:h + 1, : e - a], r["o"], r["lse"], what)
        gu.check_grads((dq[None, a:e, h:h + 1], dk[None, a:e, h:h + 1], dv[None, a:e, h:h + 1]),
                       r["grads"], what)

