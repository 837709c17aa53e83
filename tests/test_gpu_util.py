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


class _Props:
    multi_processor_count = 256


@pytest.mark.parametrize("cus", [256, 304, 80])
def test_kernel_choice_mirrors_agree(monkeypatch, cus):
    """bench.py and the GPU tests each restate fa_fwd's and fa_bwd's documented
    kernel choices; both restatements must give the same answer on every shape
    (CPU: the device's CU count is stubbed)."""
    import bench

    props = _Props()
    props.multi_processor_count = cus
    monkeypatch.setattr(torch.cuda, "get_device_properties", lambda *_: props)
    for B in (1, 2, 3, 4, 8, 16, 32, 64):
        for H in (1, 8, 13, 16, 32):
            for N in (1, 127, 128, 1000, 1024, 2048, 2500, 4096, 8192, 32768):
                for causal in (False, True):
                    fused = bench.fa_bwd_is_fused(B, H, N, causal)
                    assert fused == gu.bwd_is_fused(B, H, N, N, causal)
                    pers = gu.bwd_is_persistent(B, H, N, N, causal)
                    names = bench.fa_bwd_pass_kernel_names(B, H, N, causal)
                    if not fused:
                        assert (names[1] == "fa_bwd_dkdv_persistent_kernel") == pers[0]
                        assert (names[0] == "fa_bwd_dq_persistent_kernel") == pers[1]
                    split = bench.fa_fwd_kernel_name(B, H, N, causal) == "fa_fwd_split_kernel"
                    assert split == gu.fwd_is_key_split(B, H, N, causal)
