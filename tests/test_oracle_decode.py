"""The decoding oracle against its pins, and planted mistakes against the pins (CPU)."""

import os
import types

import pytest

import oracle
from tests import pins_decode

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "decode.py")

MUTATIONS = {
    "head_map_modulo": ("kv = h // G\n            s = _head_scores(q[b, :, h], k[b, :, kv]",
                        "kv = h % Hkv\n            s = _head_scores(q[b, :, h], k[b, :, kv]"),
    "causal_top_left": ("s = s.masked_fill(kj > qi + (nk - nq), _NEG_INF)",
                        "s = s.masked_fill(kj > qi, _NEG_INF)"),
    "causal_off_by_one": ("s = s.masked_fill(kj > qi + (nk - nq), _NEG_INF)",
                          "s = s.masked_fill(kj >= qi + (nk - nq), _NEG_INF)"),
    "scale_dropped": ("s = scale * torch.matmul(qh", "s = torch.matmul(qh"),
    "lse_missing_max": ("lse[b, h] = (m + torch.log(l)).squeeze(-1)",
                        "lse[b, h] = torch.log(l).squeeze(-1)"),
    "split_keys_unshifted": ("s = _head_scores(q[b, :, h], k[b, j0:j1, kv], scale, causal, j0, Nq, Nk)",
                             "s = _head_scores(q[b, :, h], k[b, j0:j1, kv], scale, causal, 0, Nq, Nk)"),
    "split_values_unsliced": ("o_s[b, live, h] = torch.matmul(e / l, v[b, j0:j1, kv])",
                              "o_s[b, live, h] = torch.matmul(e / l, v[b, :j1 - j0, kv])"),
    "merge_unweighted": ("o += (w_s / tot).permute(0, 2, 1).unsqueeze(-1) * o_s",
                         "o += o_s / len(partials)"),
    "merge_lse_no_shift": ("lse = safe + torch.log(tot)", "lse = torch.log(tot)"),
}


@pytest.mark.parametrize("pin", pins_decode.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


def _mutant(find, repl):
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation anchor must occur once: {find!r}"
    mod = types.ModuleType("decode_mutant")
    exec(compile(src.replace(find, repl), "decode_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in pins_decode.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or the mutant crashing outright
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin noticed mutation {name}"


def test_unmutated_copy_passes():
    mod = _mutant('_NEG_INF = float("-inf")', '_NEG_INF = float("-inf")')
    for pin in pins_decode.ALL_PINS:
        pin(mod)
