"""The CPU oracle against facts fixed outside it (CPU only)."""

import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


def test_row_chunking_is_exact():
    # Evaluating query rows in groups must reproduce the whole-matrix result.
    import torch
    g = torch.Generator().manual_seed(5)
    q, k, v, do = (torch.randn(1, 70, 2, 8, generator=g, dtype=torch.float64) for _ in range(4))
    for causal in (False, True):
        o1, l1 = oracle.attention_forward(q, k, v, 0.5, causal, row_chunk=None)
        o2, l2 = oracle.attention_forward(q, k, v, 0.5, causal, row_chunk=9)
        assert (o1 - o2).abs().max() < 1e-15 and (l1 - l2).abs().max() < 1e-15
        g1 = oracle.attention_backward(q, k, v, do, 0.5, causal, row_chunk=None)
        g2 = oracle.attention_backward(q, k, v, do, 0.5, causal, row_chunk=9)
        for a, b in zip(g1, g2):
            assert (a - b).abs().max() < 1e-13


def test_rejects_causal_rectangular():
    import torch
    q = torch.zeros(1, 4, 1, 8)
    k = torch.zeros(1, 5, 1, 8)
    with pytest.raises(ValueError):
        oracle.attention_forward(q, k, k, 1.0, True)
