"""The FP8 forward (Hadamard-rotated e4m3) on the GPU against the FP8 oracle.

Bars, per element: O max-abs <= 1e-2 + 2 * slack and LSE max-abs <= 1e-3 +
2 * slack, where slack (computed by the oracle) bounds to first order what codes
that sit at a near-tie may move -- P codes (the kernel's exponent is an fp32
value, the oracle's an fp64 one; relative tie window 2e-4 covers the matrix
unit's partial-sum rounding seen on gfx950, about 6e-6 of the largest term, times
|S| up to 30) and, end to end, Q/K codes within twice the fp32 rotation's
rounding bound of a midpoint.  Away from ties the decisions are the same.

Rows where the oracle's reference-maximum decision (the conditional rescale)
sits at a near-tie of its threshold have infinite O slack: either decision is a
correct execution.  They must stay rare (at most 1% of rows; none occur in these
cases) and keep the LSE bar.

End to end, at full size and on N(0,1) inputs the output is also held to an
a-priori error model against exact attention (tests/fp8_apriori.py): every
e4m3 rounding an independent uniform error within its half-step, propagated to
first order; |O - O_exact| <= 6 sigma + bf16 rounding.  That bound shares
nothing with the FP8 oracle, so a mistake common to the oracle and the kernel
cannot pass it.

The quantisation itself is checked code by code: the per-block scales are equal and every
code equals the oracle's, except where the oracle's value lies within the fp32
rotation bound of a midpoint, where the neighbouring code is accepted.  The
oracle's inputs never come from the GPU: the attention-stage test uploads
oracle-made codes.
"""

import math

import pytest
import torch

import oracle.fp8 as of8
from oracle import attention_forward as exact_forward
from io_aware_exact_attention_amd import fa355, workloads as wl
from tests import fp8_apriori as ap
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

TIE_REL = 2e-4
DEV = "cuda"


def _inputs(B, Nq, Nk, H, seed, outliers=False):
    x = wl.make_dense(B, Nq, H, 128, seed, Nk=Nk, with_dout=False)
    if outliers:
        # two channels of Q and K twenty times larger (the case the rotation is for)
        for n in ("q", "k"):
            t = x[n].float()
            t[..., [5, 77]] *= 20.0
            x[n] = t.to(torch.bfloat16)
    x["signs"] = wl.make_signs(128, seed + 1)
    return x


def _check(o, lse, o_ref, lse_ref, so, sl, what):
    o, lse = gu.f64(o), gu.f64(lse)
    assert torch.isfinite(o).all(), f"non-finite O {what}"
    tied = torch.isinf(so).any(-1)   # rows with a reference decision at a near-tie
    assert tied.double().mean().item() <= 0.01, f"{int(tied.sum())} near-tie rows {what}"
    eo = (o - o_ref).abs() - 2 * so
    el = (lse - lse_ref).abs() - 2 * sl
    fin = torch.isfinite(lse_ref)
    assert torch.equal(torch.isfinite(lse), fin), f"LSE finiteness {what}"
    assert eo.max().item() <= gu.O_TOL, f"O excess {eo.max().item():.3e} {what}"
    if fin.any():
        assert el[fin].max().item() <= gu.LSE_TOL, f"LSE excess {el[fin].max().item():.3e} {what}"


def _run_full(x, scale, causal, rotate=True):
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    sg = x["signs"].to(DEV)
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    ws = torch.empty(fa355.fa_fp8_workspace_bytes(B, Nq, Nk, H, d), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, Nq, dtype=torch.float32, device=DEV)
    fa355.fa_fwd_fp8(q, k, v, sg, o, lse, ws, scale, causal, rotate)
    torch.cuda.synchronize()
    return o, lse, ws


CASES = [
    # B, Nq, Nk, H, causal
    (1, 300, 300, 2, True),      # several tiles and a ragged tail
    (2, 257, 257, 3, False),
    (1, 64, 64, 1, True),        # exactly one tile
    (2, 77, 200, 2, False),      # Nq != Nk
    (1, 1, 1, 2, True),          # a single token
    (1, 1, 513, 2, False),       # one query, many keys
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Nq{}_Nk{}_H{}_{}".format(
    *c[:4], "causal" if c[4] else "full"))
def test_fp8_quantisation_codes(case):
    gu.need_gpu()
    B, Nq, Nk, H, causal = case
    gu.announce(f"fp8 quantise B{B} Nq{Nq} Nk{Nk} H{H}")
    x = _inputs(B, Nq, Nk, H, seed=3000 + Nq + Nk + H)
    _, _, ws = _run_full(x, 128 ** -0.5, causal)
    q8, k8, v8, scales = fa355.fp8_workspace_views(ws, B, Nq, Nk, H, 128)
    for t, (name, sg) in enumerate((("q", x["signs"]), ("k", x["signs"]), ("v", None))):
        codes_ref, s_ref, scaled = of8.quantize_e4m3(x[name], sg)
        got = [q8, k8, v8][t].cpu()
        assert torch.equal(gu.f64(scales[t][..., :s_ref.shape[-1]]), s_ref), f"{name} scales"
        diff = got != codes_ref
        if diff.any():
            assert sg is not None, f"{name}: unrotated values are exact, codes must match"
            atol = 2.0 * of8.fp32_rotation_error(x[name], sg, s_ref)
            tie = of8.e4m3_near_tie(scaled, 1e-7, atol)
            assert bool(tie[diff].all()), f"{name}: {int((diff & ~tie).sum())} codes differ off a tie"
            # and the accepted ones are the neighbouring code of the same sign
            dv = (of8.e4m3_decode(got[diff]) - of8.e4m3_decode(codes_ref[diff])).abs()
            assert bool((dv <= of8.e4m3_step(codes_ref[diff]) + of8.e4m3_step(got[diff])).all())


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Nq{}_Nk{}_H{}_{}".format(
    *c[:4], "causal" if c[4] else "full"))
def test_fp8_attention_stage(case):
    # the attention kernel alone, on codes and scales the oracle made
    gu.need_gpu()
    B, Nq, Nk, H, causal = case
    gu.announce(f"fp8 attention codes B{B} Nq{Nq} Nk{Nk} H{H} causal={causal}")
    x = _inputs(B, Nq, Nk, H, seed=3100 + Nq + Nk + H)
    q8, sq, _ = of8.quantize_e4m3(x["q"], x["signs"])
    k8, sk, _ = of8.quantize_e4m3(x["k"], x["signs"])
    v8, sv, _ = of8.quantize_e4m3(x["v"], None)
    qk_scale = 128 ** -0.5 / 128
    o_ref, lse_ref, so, sl = of8.fp8_attention_forward(q8, k8, v8, sq, sk, sv, qk_scale, causal, TIE_REL)
    dev = [t.to(DEV) for t in (q8, k8, v8)]
    sc = [t.to(torch.float32).reshape(-1).to(DEV) for t in (sq, sk, sv)]
    o = torch.empty(B, Nq, H, 128, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, H, Nq, dtype=torch.float32, device=DEV)
    fa355.fa_fwd_fp8_codes(*dev, *sc, o, lse, qk_scale, causal)
    torch.cuda.synchronize()
    _check(o, lse, o_ref, lse_ref, so, sl, f"codes {case}")


def test_fp8_attention_stage_both_rescale_paths():
    # K three times larger (the long-context recipe): the row maxima rise after
    # the first key tile by more than ln 16 in some rows (the reference moves and
    # O is rescaled) and by less in others (the reference stays, P~ up to 16)
    gu.need_gpu()
    B, N, H = 1, 1024, 2
    gu.announce(f"fp8 attention codes, both rescale paths, B{B} N{N} H{H} K x3")
    x = _inputs(B, N, N, H, seed=3400)
    x["k"] = (x["k"].float() * 3.0).to(torch.bfloat16)
    q8, sq, _ = of8.quantize_e4m3(x["q"], x["signs"])
    k8, sk, _ = of8.quantize_e4m3(x["k"], x["signs"])
    v8, sv, _ = of8.quantize_e4m3(x["v"], None)
    qk_scale = 128 ** -0.5 / 128
    # the case has both kinds of rows (scores of the decoded codes, causal)
    qd = of8.e4m3_decode(q8) * of8.row_scales(sq, N, 64).transpose(1, 2)[..., None]
    kd = of8.e4m3_decode(k8) * of8.row_scales(sk, N, 64).transpose(1, 2)[..., None]
    sc = qk_scale * torch.einsum("bihd,bjhd->bhij", qd, kd)
    sc = sc.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    rise = (sc.amax(-1) - sc[..., :64].amax(-1))[..., 64:]   # rows that see a second tile
    thr = 4 * math.log(2.0)
    assert int((rise > thr).sum()) > 50 and int(((rise > 0) & (rise < thr)).sum()) > 50
    o_ref, lse_ref, so, sl = of8.fp8_attention_forward(q8, k8, v8, sq, sk, sv, qk_scale, True, TIE_REL)
    dev = [t.to(DEV) for t in (q8, k8, v8)]
    scl = [t.to(torch.float32).reshape(-1).to(DEV) for t in (sq, sk, sv)]
    o = torch.empty(B, N, H, 128, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=DEV)
    fa355.fa_fwd_fp8_codes(*dev, *scl, o, lse, qk_scale, True)
    torch.cuda.synchronize()
    _check(o, lse, o_ref, lse_ref, so, sl, "both rescale paths")


@pytest.mark.parametrize("case", CASES[:4], ids=lambda c: "B{}_Nq{}_Nk{}_H{}_{}".format(
    *c[:4], "causal" if c[4] else "full"))
@pytest.mark.parametrize("rotate", [True, False], ids=["rotated", "plain"])
def test_fp8_end_to_end(case, rotate):
    gu.need_gpu()
    B, Nq, Nk, H, causal = case
    gu.announce(f"fp8 end to end B{B} Nq{Nq} Nk{Nk} H{H} causal={causal} rotate={rotate}")
    x = _inputs(B, Nq, Nk, H, seed=3200 + Nq + Nk + H)
    scale = 128 ** -0.5
    o, lse, _ = _run_full(x, scale, causal, rotate)
    o_ref, lse_ref, so, sl, _, _ = of8.fp8_forward(x["q"], x["k"], x["v"], x["signs"], scale, causal,
                                                   rotate, TIE_REL, fp32_rotation=True)
    _check(o, lse, o_ref, lse_ref, so, sl, f"end to end {case} rotate={rotate}")
    # and against exact attention, within the a-priori e4m3 error model (which
    # shares nothing with the FP8 oracle's algorithm or design choices)
    ref = ap.fp8_sigma(x["q"], x["k"], x["v"], x["signs"], scale, causal, rotate)
    r_o, r_l, rms, outside = ap.check_apriori(o, lse, *ref, what=f"end to end {case} rotate={rotate}")
    assert outside == 0.0


def test_fp8_deterministic():
    gu.need_gpu()
    x = _inputs(2, 700, 700, 2, seed=33)
    a = _run_full(x, 0.088, True)
    b = _run_full(x, 0.088, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # the codes and scales (the workspace's padding and block maxima are scratch)
    for u, w in zip(fa355.fp8_workspace_views(a[2], 2, 700, 700, 2, 128),
                    fa355.fp8_workspace_views(b[2], 2, 700, 700, 2, 128)):
        assert torch.equal(u, w)


def test_fp8_error_against_exact_and_rotation_helps():
    # the page's point, on the GPU path: with outlier channels in Q and K, the
    # rotated FP8 forward is closer to exact attention than the unrotated one
    gu.need_gpu()
    gu.announce("fp8 rmse vs exact, outliers")
    B, N, H = 1, 512, 4
    scale = 0.02
    x = _inputs(B, N, N, H, seed=3300, outliers=True)
    o_ex, _ = exact_forward(x["q"], x["k"], x["v"], scale, True)
    o_rot = _run_full(x, scale, True, True)[0]
    o_pl = _run_full(x, scale, True, False)[0]
    e_rot, e_pl = of8.rmse(o_rot, o_ex), of8.rmse(o_pl, o_ex)
    print(f"[fp8] rmse vs exact: rotated {e_rot:.3e}, unrotated {e_pl:.3e}", flush=True)
    assert e_rot < e_pl
    # and without outliers every element of the FP8 forward lies within the
    # a-priori e4m3 error model's bound of exact attention
    y = _inputs(B, N, N, H, seed=3301)
    o2, lse2, _ = _run_full(y, 128 ** -0.5, True, True)
    ref = ap.fp8_sigma(y["q"], y["k"], y["v"], y["signs"], 128 ** -0.5, True, True)
    r_o, r_l, rms, outside = ap.check_apriori(o2, lse2, *ref, what="N(0,1) inputs")
    print(f"[fp8] N(0,1) inputs: rmse vs exact {of8.rmse(o2, ref[0]):.3e}; largest error "
          f"{r_o:.2f} (O) / {r_l:.2f} (LSE) of the a-priori bound, rms error/sigma {rms:.2f}", flush=True)
    assert outside == 0.0


def test_fp8_workload_full_size_sampled():
    # the benchmarked shape at full size; whole (batch, head) slices compared
    gu.need_gpu()
    w8 = wl.FP8_WORKLOADS["fp8_b8_h16_n4096_d128_causal"]
    base = wl.WORKLOADS[w8.base]
    gu.announce(f"fp8 full size {w8.name}")
    x = wl.make_inputs(w8.name)
    o, lse, ws = _run_full(x, base.scale, True)
    assert torch.isfinite(o).all()
    for b, h in ((0, 0), (5, 11)):
        sl_ = slice(h, h + 1)
        o_ref, lse_ref, so, sl, _, _ = of8.fp8_forward(
            x["q"][b:b + 1, :, sl_], x["k"][b:b + 1, :, sl_], x["v"][b:b + 1, :, sl_], x["signs"],
            base.scale, True, True, TIE_REL, fp32_rotation=True)
        _check(o[b:b + 1, :, sl_], lse[b:b + 1, sl_], o_ref, lse_ref, so, sl, f"full size b{b} h{h}")
        ref = ap.fp8_sigma(x["q"][b:b + 1, :, sl_], x["k"][b:b + 1, :, sl_], x["v"][b:b + 1, :, sl_],
                           x["signs"], base.scale, True, True)
        ap.check_apriori(o[b:b + 1, :, sl_], lse[b:b + 1, sl_], *ref, what=f"full size b{b} h{h}")


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_fp8_rows_past_a_sequence_read_as_zeros(causal):
    """Batch entry 1 is all NaN (its quantisation scales and codes are NaN); the
    tiles of batch entry 0 that run past its 77 rows must read zeros, not those."""
    gu.need_gpu()
    gu.announce(f"fp8 NaN neighbours causal={causal}")
    x = _inputs(2, 77, 77, 2, seed=3900)
    xn = {n: (t.clone() if n != "signs" else t) for n, t in x.items()}
    for n in ("q", "k", "v"):
        xn[n][1] = float("nan")
    scale = 128 ** -0.5
    o, lse, _ = _run_full(xn, scale, causal)
    o_ref, lse_ref, so, sl, _, _ = of8.fp8_forward(x["q"][:1], x["k"][:1], x["v"][:1], x["signs"], scale,
                                                   causal, True, TIE_REL, fp32_rotation=True)
    _check(o[:1], lse[:1], o_ref, lse_ref, so, sl, "fp8 batch 0 with NaN neighbours")
