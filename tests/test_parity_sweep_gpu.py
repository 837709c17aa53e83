"""A seeded sweep of random small shapes through every entry point (GPU vs oracle).

Shapes are drawn once from a fixed seed (sizes up to a few tiles, ragged tails,
Nq != Nk where allowed, both head dims, both masks, batch and head counts that
are and are not multiples of 8), so that corner combinations the hand-picked
cases miss are still compared element by element at the same bounds.
"""

import random

import pytest
import torch

import oracle
import oracle.fp8 as of8
from io_aware_exact_attention_amd import fa355, workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _dense_cases(n=12, seed=5150):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        causal = rng.random() < 0.5
        nq = rng.choice([1, 2, 31, 33, 64, 127, 128, 129, 191, 257, 300, 400])
        nk = nq if causal else rng.choice([1, 5, 63, 64, 65, 200, 333, 512])
        out.append((rng.choice([1, 2, 3]), nq, nk, rng.choice([1, 2, 5, 8]), rng.choice([64, 128]), causal))
    return out


def _ids(c):
    return "B{}_Nq{}_Nk{}_H{}_d{}_{}".format(*c[:5], "causal" if c[5] else "full")


@pytest.mark.parametrize("case", _dense_cases(), ids=_ids)
def test_sweep_dense_fwd_bwd_persistent(case):
    gu.need_gpu()
    B, Nq, Nk, H, d, causal = case
    gu.announce(f"sweep dense {case}")
    x = wl.make_dense(B, Nq, H, d, seed=9000 + Nq * 7 + Nk + H + d, Nk=Nk)
    scale = d ** -0.5
    g = gu.run_dense(x, scale, causal)
    r = gu.oracle_dense(x, scale, causal)
    gu.check_forward(g["o"], g["lse"], r["o"], r["lse"], str(case))
    gu.check_grads(g["grads"], r["grads"], str(case))
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o2 = torch.empty_like(q)
    l2 = torch.empty(B, H, Nq, dtype=torch.float32, device=q.device)
    fa355.fa_fwd_persistent(q, k, v, o2, l2, scale, causal)
    torch.cuda.synchronize()
    if gu.fwd_is_key_split(B, H, Nq, causal):
        gu.check_forward(o2, l2, r["o"], r["lse"], f"persistent {case}")
    else:
        assert torch.equal(o2.cpu(), g["o"].cpu()) and torch.equal(l2.cpu(), g["lse"].cpu())


def _dense_cases_large(n=8, seed=5152):
    """Shapes large enough that some take the one-tile-per-work-group forward and
    the two-kernel backward (grids beyond a few work-groups per CU), with ragged
    tails, alongside ones that take the key-split forward and one-launch backward."""
    out = [
        (3, 1900, 1900, 32, 128, True),    # one-tile forward, two-kernel backward (256 CUs)
        (2, 1500, 1300, 16, 64, False),    # persistent forward, two-kernel backward
        (2, 2100, 2100, 24, 64, True),     # one-tile forward, one-launch backward
    ]
    rng = random.Random(seed)
    for _ in range(n):
        causal = rng.random() < 0.6
        nq = rng.choice([600, 1000, 1500, 2048, 2500])
        nk = nq if causal else rng.choice([700, 1100, 2049])
        out.append((rng.choice([1, 2]), nq, nk, rng.choice([4, 8, 12, 16]), rng.choice([64, 128]), causal))
    return out


@pytest.mark.parametrize("case", _dense_cases_large(), ids=_ids)
def test_sweep_dense_large(case):
    gu.need_gpu()
    B, Nq, Nk, H, d, causal = case
    gu.announce(f"sweep dense large {case}")
    x = wl.make_dense(B, Nq, H, d, seed=9300 + Nq * 3 + Nk + H + d, Nk=Nk)
    scale = d ** -0.5
    g = gu.run_dense(x, scale, causal)
    r = gu.oracle_dense(x, scale, causal)
    gu.check_forward(g["o"], g["lse"], r["o"], r["lse"], str(case))
    gu.check_grads(g["grads"], r["grads"], str(case))


def _decode_cases(n=6, seed=5151):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        hkv = rng.choice([1, 2, 4])
        G = rng.choice([1, 2, 4, 8, 16])
        nq = rng.choice([1, 2, 3, 4])
        nk = rng.choice([nq, 33, 100, 1000, 5000])
        out.append((rng.choice([1, 2]), nq, max(nk, nq), hkv * G, hkv, rng.choice([64, 128]), rng.random() < 0.5))
    return out


@pytest.mark.parametrize("case", _decode_cases(), ids=lambda c: "B{}_Nq{}_Nk{}_Hq{}_Hkv{}_d{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
def test_sweep_decode(case):
    gu.need_gpu()
    B, Nq, Nk, Hq, Hkv, d, causal = case
    gu.announce(f"sweep decode {case}")
    y = wl.make_decode(B, Nq, Nk, Hq, Hkv, d, seed=9100 + Nk + Hq)
    scale = d ** -0.5
    o, lse = fa355.attention_decode(y["q"].cuda(), y["k"].cuda(), y["v"].cuda(), scale, causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_forward(y["q"], y["k"], y["v"], scale, causal)
    gu.check_forward(o, lse, o_ref, lse_ref, str(case))


def _fp8_cases(n=6, seed=5152):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        causal = rng.random() < 0.5
        nq = rng.choice([1, 63, 65, 130, 256, 333])
        nk = nq if causal else rng.choice([1, 64, 99, 257])
        out.append((rng.choice([1, 2]), nq, nk, rng.choice([1, 3, 8]), causal, rng.random() < 0.7))
    return out


@pytest.mark.parametrize("case", _fp8_cases(), ids=lambda c: "B{}_Nq{}_Nk{}_H{}_{}_{}".format(
    *c[:4], "causal" if c[4] else "full", "rot" if c[5] else "plain"))
def test_sweep_fp8(case):
    gu.need_gpu()
    B, Nq, Nk, H, causal, rotate = case
    gu.announce(f"sweep fp8 {case}")
    x = wl.make_dense(B, Nq, H, 128, seed=9200 + Nq + Nk + H, Nk=Nk, with_dout=False)
    sg = wl.make_signs(128, 9201 + H)
    scale = 128 ** -0.5
    o, lse = fa355.attention_forward_fp8(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), sg.cuda(), scale,
                                         causal, rotate)
    torch.cuda.synchronize()
    o_ref, lse_ref, so, sl, _, _ = of8.fp8_forward(x["q"], x["k"], x["v"], sg, scale, causal, rotate,
                                                   2e-4, fp32_rotation=True)
    eo = ((gu.f64(o) - o_ref).abs() - 2 * so).max().item()
    el = ((gu.f64(lse) - lse_ref).abs() - 2 * sl).max().item()
    assert eo <= gu.O_TOL and el <= gu.LSE_TOL, (eo, el)
