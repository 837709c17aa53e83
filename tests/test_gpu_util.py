"""The parity helpers' own rules, on hand-made values (CPU)."""

import pytest
import torch

from tests import gpu_util as gu


def test_bf16_ulp():
    x = torch.tensor([1.0, 1.5, 2.0, 3.99, 4.0, 4.107, -5.0, 0.75], dtype=torch.float64)
    want = [2 ** -7, 2 ** -7, 2 ** -6, 2 ** -6, 2 ** -5, 2 ** -5, 2 ** -5, 2 ** -8]
    assert gu.bf16_ulp(x).tolist() == want


def _fwd(o_gpu, o_ref):
    lse = torch.zeros(1, 1, 1, dtype=torch.float64)
    return gu.check_forward(torch.tensor(o_gpu, dtype=torch.float64).reshape(1, 1, 1, -1), lse,
                            torch.tensor(o_ref, dtype=torch.float64).reshape(1, 1, 1, -1), lse)


def test_o_tolerance_and_output_floor():
    # |O| < 4: the literal 1e-2 bound holds for every entry
    _fwd([3.0, 1.0], [3.0 + 0.0099, 1.0])
    with pytest.raises(AssertionError):
        _fwd([3.0, 1.0], [3.0 + 0.0101, 1.0])
    # 4.0105 lies 0.0105 from its nearest bf16 value (4.0): its own floor exceeds
    # 1e-2, so it is held to one bf16 step (2^-5) instead
    _fwd([4.0, 1.0], [4.0105, 1.0])
    _fwd([4.03125, 1.0], [4.0105, 1.0])
    with pytest.raises(AssertionError):
        _fwd([4.0625, 1.0], [4.0105, 1.0])
    # 4.005 has a floor of 0.005: the 1e-2 bound applies to it
    with pytest.raises(AssertionError):
        _fwd([4.03125, 1.0], [4.005, 1.0])
    # a floor-limited entry does not excuse another entry's error
    with pytest.raises(AssertionError):
        _fwd([4.0, 1.02], [4.0105, 1.0])
