"""The FP8 oracle against its pins, and planted mistakes against the pins (CPU)."""

import os
import types

import pytest

import oracle.fp8 as fp8
from tests import pins_fp8

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "fp8.py")

MUTATIONS = {
    "decode_bias_8": ("normal = torch.ldexp(1.0 + m / 8.0, (e - 7).to(torch.float64))",
                      "normal = torch.ldexp(1.0 + m / 8.0, (e - 8).to(torch.float64))"),
    "decode_subnormal_exponent": ("sub = torch.ldexp(m / 8.0, torch.full_like(m, -6.0))",
                                  "sub = torch.ldexp(m / 8.0, torch.full_like(m, -7.0))"),
    "encode_ties_away": ("q = torch.round(a / quantum) * quantum",
                         "q = torch.floor(a / quantum + 0.5) * quantum"),
    "encode_truncates": ("q = torch.round(a / quantum) * quantum",
                         "q = torch.floor(a / quantum) * quantum"),
    "encode_no_saturation": ("a = x.abs().clamp(max=E4M3_MAX)\n    # spacing",
                             "a = x.abs()\n    # spacing"),
    "encode_subnormal_spacing": ("e = _binade(a).clamp(min=-6.0)", "e = _binade(a).clamp(min=-7.0)"),
    "encode_drops_sign": ("code = torch.where(torch.signbit(x), code | 128, code)", "code = code"),
    "hadamard_not_orthogonal": ("h = torch.cat([torch.cat([h, h], 1), torch.cat([h, -h], 1)], 0)",
                                "h = torch.cat([torch.cat([h, h], 1), torch.cat([-h, h], 1)], 0)"),
    "rotate_ignores_signs": ("return torch.matmul(x * _f64(signs).reshape(d), hadamard(d))",
                             "return torch.matmul(x, hadamard(d))"),
    "rotate_transposed_signs": ("return torch.matmul(x * _f64(signs).reshape(d), hadamard(d))",
                                "return torch.matmul(x, hadamard(d)) * _f64(signs).reshape(d)"),
    "scale_not_power_of_two": ("s = torch.where(amax > 0, torch.ldexp(torch.ones_like(amax), e), torch.ones_like(amax))",
                               "s = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))"),
    "scale_rounds_down": ("e = torch.ceil(torch.log2(", "e = torch.floor(torch.log2("),
    "scores_missing_k_scale": ("c = qk_scale * torch.outer(rq[b, h], rk[b, h])",
                               "c = qk_scale * rq[b, h][:, None] * torch.ones_like(rk[b, h])[None, :]"),
    "scores_scales_swapped": ("c = qk_scale * torch.outer(rq[b, h], rk[b, h])",
                              "c = qk_scale * torch.outer(rk[b, h][:Nq], rq[b, h][:Nk]) if Nq == Nk else qk_scale * torch.outer(rq[b, h], rk[b, h])"),
    "block_scales_shifted": ("return s.repeat_interleave(int(rows), dim=2)[:, :, :n]",
                             "return s.repeat_interleave(int(rows), dim=2)[:, :, 1:n + 1] if s.shape[2] * int(rows) > n else s.repeat_interleave(int(rows), dim=2)[:, :, :n]"),
    "quantise_per_head": ("rows = N if block_rows is None else int(block_rows)\n    nblk",
                          "rows = N\n    nblk"),
    "p_scale_not_undone": ("o[b, :, h] = acc / p_scale * linv", "o[b, :, h] = acc * linv"),
    "v_scale_dropped": ("vh = vd[b, :, h] * rv[b, h][:, None]", "vh = vd[b, :, h]"),
    "p_not_quantised": ("p8 = e4m3_encode(p_scale * pt)\n                pq = e4m3_decode(p8)",
                        "p8 = e4m3_encode(p_scale * pt)\n                pq = p_scale * pt"),
    "p_rounded_at_final_max": ("p8 = e4m3_encode(p_scale * pt)\n                pq = e4m3_decode(p8)",
                               "p8 = e4m3_encode(p_scale * torch.exp(sb - m_fin0))\n"
                               "                pq = e4m3_decode(p8) * torch.exp(m_fin0 - m_ref)"),
    "p_scale_fixed_256": ("p_scale = 2.0 ** (8.0 - rescale_log2)", "p_scale = 256.0"),
    "rescale_always": ("m_new = torch.where(m_blk > m + thr, m_blk, m)", "m_new = torch.maximum(m, m_blk)"),
    "threshold_natural_units": ("thr = rescale_log2 * math.log(2.0)", "thr = rescale_log2"),
    "threshold_not_strict_sign": ("m_new = torch.where(m_blk > m + thr, m_blk, m)",
                                  "m_new = torch.where(m_blk > m - thr, m_blk, m)"),
    "alpha_from_block_max": ("alpha = torch.exp(m - m_ref)", "alpha = torch.exp(m - torch.maximum(m_ref, m_blk))"),
    "slack_at_true_maximum": ("tie_p = alpha * tie_p + torch.matmul(tp, vh[j0:j0 + bs].abs())",
                              "tie_p = alpha * tie_p + torch.exp(m_ref - m_fin0) * torch.matmul(tp, vh[j0:j0 + bs].abs())"),
    "near_tie_not_flagged": ("amb |= fin & ((rise - thr).abs() <= tie_rel * (m.abs() + m_blk.abs()))",
                             "amb |= fin & ((rise - thr).abs() < 0.0)"),
    "near_tie_flags_everything": ("amb |= fin & ((rise - thr).abs() <= tie_rel * (m.abs() + m_blk.abs()))",
                                  "amb |= fin"),
    "acc_not_rescaled": ("acc = alpha * acc + torch.matmul(pq, vh[j0:j0 + bs])",
                         "acc = acc + torch.matmul(pq, vh[j0:j0 + bs])"),
    "sum_not_rescaled": ("l = alpha * l + pt.sum(dim=-1, keepdim=True)",
                         "l = l + pt.sum(dim=-1, keepdim=True)"),
    "block_offset_ignored": ("acc = alpha * acc + torch.matmul(pq, vh[j0:j0 + bs])",
                             "acc = alpha * acc + torch.matmul(pq, vh[0:sb.shape[1]])"),
    "causal_off_by_one": ("vis = torch.arange(Nk).unsqueeze(0) <= torch.arange(Nq).unsqueeze(1)",
                          "vis = torch.arange(Nk).unsqueeze(0) < torch.arange(Nq).unsqueeze(1)"),
    "lse_missing_max": ("lse[b, h] = torch.where(live, m + torch.log(l),",
                        "lse[b, h] = torch.where(live, torch.log(l),"),
    "rotation_norm_missing": ("qk_scale = scale / d if rotate_qk else scale",
                              "qk_scale = scale"),
    "v_rotated_too": ("v8, sv, vs = quantize_e4m3(v, None)", "v8, sv, vs = quantize_e4m3(v, sg)"),
    # the slack's own terms and the rotation's rounding bound
    "rotation_error_no_log2d": ("return math.log2(d) * 2.0 ** -24 * l1", "return 2.0 ** -24 * l1"),
    "rotation_error_x4": ("return math.log2(d) * 2.0 ** -24 * l1", "return 4 * math.log2(d) * 2.0 ** -24 * l1"),
    "rotation_error_x2": ("return math.log2(d) * 2.0 ** -24 * l1", "return 2 * math.log2(d) * 2.0 ** -24 * l1"),
    "rotation_error_ignores_scale": ("l1 / row_scales(s, N, block_rows).transpose(1, 2)[..., None]", "l1"),
    "rotation_error_fp64_eps": ("return math.log2(d) * 2.0 ** -24 * l1", "return math.log2(d) * 2.0 ** -53 * l1"),
    "slack_drops_ds": ("so + dev)", "so)"),
    "slack_o_x4": ("so + dev)", "4 * (so + dev))"),
    "slack_l_x4": ("slack_l[b, h] = (p_true * ds).sum(dim=-1)", "slack_l[b, h] = 4 * (p_true * ds).sum(dim=-1)"),
    "slack_l_dropped": ("slack_l[b, h] = (p_true * ds).sum(dim=-1)", "slack_l[b, h] = 0.0 * (p_true * ds).sum(dim=-1)"),
    "slack_drops_tie_v": ("so = (tie_p + tie_v) / p_scale * linv", "so = tie_p / p_scale * linv"),
    "slack_drops_tie_p": ("so = (tie_p + tie_v) / p_scale * linv", "so = tie_v / p_scale * linv"),
    "k_ties_ignored": ("tq, tk = tie_steps(q_scaled, q8, q_tie_atol), tie_steps(k_scaled, k8, k_tie_atol)",
                       "tq, tk = tie_steps(q_scaled, q8, q_tie_atol), tie_steps(None, k8)"),
    "q_ties_ignored": ("tq, tk = tie_steps(q_scaled, q8, q_tie_atol), tie_steps(k_scaled, k8, k_tie_atol)",
                       "tq, tk = tie_steps(None, q8), tie_steps(k_scaled, k8, k_tie_atol)"),
    "ds_k_signed": ("torch.matmul(tq[b, :, h], kh.abs().transpose(0, 1))", "torch.matmul(tq[b, :, h], kh.transpose(0, 1))"),
    "ds_q_signed": ("torch.matmul(qh.abs(), tk[b, :, h].transpose(0, 1))", "torch.matmul(qh, tk[b, :, h].transpose(0, 1))"),
    "dev_drops_o_term": ("dev = torch.matmul(p_true * ds, vabs) + (p_true * ds).sum(-1, keepdim=True) * o[b, :, h].abs()",
                         "dev = torch.matmul(p_true * ds, vabs)"),
    "tie_v_unscaled": ("tvh = tv[b, :, h] * rv[b, h][:, None]", "tvh = tv[b, :, h]"),
}


@pytest.mark.parametrize("pin", pins_fp8.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(fp8)


def _mutant(find, repl):
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation anchor must occur once: {find!r}"
    mod = types.ModuleType("fp8_mutant")
    exec(compile(src.replace(find, repl), "fp8_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in pins_fp8.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or the mutant crashing outright
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin noticed mutation {name}"


def test_unmutated_copy_passes():
    mod = _mutant('_NEG_INF = float("-inf")', '_NEG_INF = float("-inf")')
    for pin in pins_fp8.ALL_PINS:
        pin(mod)
