"""The a-priori e4m3 error model (tests/fp8_apriori.py) on the CPU: it covers
the FP8 oracle's error against exact attention and is not loose (the RMS of
error / sigma is near 1), and it rejects the FP8 oracle with mistakes planted
that the kernel could share (so the GPU tests' gate against exact attention
catches them independently of the oracle).  A different orthogonal rotation
(no random signs) is no such mistake: it leaves the scores and the accuracy as
they are, and the oracle's own pins catch it."""

import os
import types

import pytest
import torch

import oracle.fp8 as of8
from io_aware_exact_attention_amd import workloads as wl
from tests import fp8_apriori as ap

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "fp8.py")


def _case(seed, n=192, causal=True, kscale=1.0):
    x = wl.make_dense(1, n, 2, 128, seed=seed, with_dout=False)
    if kscale != 1.0:
        x["k"] = (x["k"].float() * kscale).to(torch.bfloat16)
    x["signs"] = wl.make_signs(128, seed + 1)
    return x


@pytest.mark.parametrize("causal,kscale,rotate", [(True, 1.0, True), (False, 1.0, True),
                                                  (True, 3.0, True), (True, 1.0, False)])
def test_model_covers_the_fp8_oracle_and_is_tight(causal, kscale, rotate):
    x = _case(501, causal=causal, kscale=kscale)
    scale = 128 ** -0.5
    ref = ap.fp8_sigma(x["q"], x["k"], x["v"], x["signs"], scale, causal, rotate)
    o, lse, *_ = of8.fp8_forward(x["q"], x["k"], x["v"], x["signs"], scale, causal, rotate)
    r_o, r_l, rms, outside = ap.check_apriori(o, lse, *ref)
    assert outside == 0.0
    assert 0.4 <= rms <= 1.3, rms          # the model's sigma is the error's own scale
    assert r_o >= 0.2, r_o                 # and the 6-sigma bound is not loose by orders


MISTAKES = {
    "rotation_norm_missing": ("qk_scale = scale / d if rotate_qk else scale", "qk_scale = scale"),
    "v_rotated_too": ("v8, sv, vs = quantize_e4m3(v, None)", "v8, sv, vs = quantize_e4m3(v, sg)"),
    "p_scale_not_undone": ("o[b, :, h] = acc / p_scale * linv", "o[b, :, h] = acc * linv"),
    "v_scale_dropped": ("vh = vd[b, :, h] * rv[b, h][:, None]", "vh = vd[b, :, h]"),
    "k_scale_missing": ("c = qk_scale * torch.outer(rq[b, h], rk[b, h])",
                        "c = qk_scale * rq[b, h][:, None] * torch.ones_like(rk[b, h])[None, :]"),
    "causal_off_by_one": ("vis = torch.arange(Nk).unsqueeze(0) <= torch.arange(Nq).unsqueeze(1)",
                          "vis = torch.arange(Nk).unsqueeze(0) < torch.arange(Nq).unsqueeze(1)"),
    "sum_not_rescaled": ("l = alpha * l + pt.sum(dim=-1, keepdim=True)", "l = l + pt.sum(dim=-1, keepdim=True)"),
    "p_truncated": ("p8 = e4m3_encode(p_scale * pt)", "p8 = e4m3_encode(torch.floor(p_scale * pt))"),
}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_model_rejects_a_shared_mistake(name):
    find, repl = MISTAKES[name]
    src = open(SRC).read()
    assert src.count(find) == 1, find
    mod = types.ModuleType("fp8_mistake")
    exec(compile(src.replace(find, repl), "fp8_mistake", "exec"), mod.__dict__)
    x = _case(502, n=256, kscale=3.0)   # K x3: row maxima rise past the rescale threshold
    scale = 128 ** -0.5
    ref = ap.fp8_sigma(x["q"], x["k"], x["v"], x["signs"], scale, True, True)
    o, lse, *_ = mod.fp8_forward(x["q"], x["k"], x["v"], x["signs"], scale, True, True)
    with pytest.raises(AssertionError):
        ap.check_apriori(o, lse, *ref)
