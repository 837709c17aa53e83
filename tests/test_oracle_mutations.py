"""Plant plausible mistakes in a copy of the oracle and check that the pins notice.

Each mutation edits the oracle's source text once (on the CPU, in a private
module object) and runs every pin; at least one pin must fail.  This keeps
the pins honest: a dropped term, a wrong sign or index, or a transposed
operand anywhere in the oracle is caught.
"""

import os
import types

import pytest

from tests import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "attention.py")

MUTATIONS = {
    "no_max_subtraction": ("e = torch.exp(s - m)", "e = torch.exp(s)"),
    "scale_dropped": ("s = scale * torch.matmul(q_rows", "s = torch.matmul(q_rows"),
    "causal_off_by_one": ("s = s.masked_fill(kj > qi, _NEG_INF)\n    return s",
                          "s = s.masked_fill(kj >= qi, _NEG_INF)\n    return s"),
    "causal_chunk_drops_last_key": ("kend = r1 if causal else kb.shape[1]",
                                    "kend = r1 - 1 if causal else kb.shape[1]"),
    "lse_log2": ("lse[b, :, r0:r1] = m + torch.log(l)", "lse[b, :, r0:r1] = m + torch.log2(l)"),
    "lse_missing_max": ("lse[b, :, r0:r1] = m + torch.log(l)", "lse[b, :, r0:r1] = torch.log(l)"),
    "dv_untransposed_p": ("dvb[:, :kend] += torch.matmul(p.transpose(-1, -2), do_r)",
                          "dvb[:, :kend] += torch.matmul(p.transpose(-1, -2), dob[:, r0:r1] * 0.5)"),
    "ds_wrong_sign": ("ds = p * (dp - drow)", "ds = p * (dp + drow)"),
    "ds_missing_d": ("ds = p * (dp - drow)", "ds = p * dp"),
    "dq_uses_p": ("torch.matmul(ds, kb[:, :kend])", "torch.matmul(p, kb[:, :kend])"),
    "dk_missing_scale": ("dkb[:, :kend] += scale * torch.matmul", "dkb[:, :kend] += torch.matmul"),
    "dk_uses_dq_operand": ("torch.matmul(ds.transpose(-1, -2), qb[:, r0:r1])",
                           "torch.matmul(ds.transpose(-1, -2), kb[:, r0:r1])"),
    "d_vector_wrong": ("drow = (p * dp).sum(dim=-1, keepdim=True)",
                       "drow = dp.sum(dim=-1, keepdim=True) / dp.shape[-1]"),
    "online_sum_not_rescaled": ("l = f_old * l + f_blk * l_blk", "l = l + f_blk * l_blk"),
    "online_acc_not_rescaled": ("acc = f_old.unsqueeze(-1) * acc", "acc = acc"),
    "online_block_factor_dropped": ("+ f_blk.unsqueeze(-1) * torch.matmul(p_t",
                                    "+ torch.matmul(p_t"),
    "online_causal_mask_flipped": ("s = s.masked_fill(kj > qi, _NEG_INF)\n            m_blk",
                                   "s = s.masked_fill(kj < qi, _NEG_INF)\n            m_blk"),
    "varlen_wrong_key_slice": ("k[None, k0:k1], v[None, k0:k1],\n                                     scale",
                               "k[None, q0:q1], v[None, k0:k1],\n                                     scale"),
}


def _mutant(find, repl):
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation anchor must occur once: {find!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(find, repl), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or the mutant crashing outright
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin noticed mutation {name}"


def test_unmutated_copy_passes():
    mod = _mutant("_NEG_INF = float(\"-inf\")", "_NEG_INF = float(\"-inf\")")
    for pin in pins.ALL_PINS:
        pin(mod)
