"""The persistent, longest-first forward (fa_fwd_persistent) on the GPU: bitwise
equal to fa_fwd wherever fa_fwd runs the per-tile or persistent kernel (each tile
is the same computation, only the work-group that runs it differs), and to the
oracle within the forward's bounds.  Small causal grids, where fa_fwd runs the
key-split kernel instead, are compared with the oracle directly."""

import pytest
import torch

import oracle
from io_aware_exact_attention_amd import fa355, workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    # B, N, Nk, H, d, causal
    (2, 1000, 1000, 8, 128, True),     # B*H a multiple of 8: XCD-dealt pairs
    (1, 300, 300, 3, 64, True),        # B*H not a multiple of 8, ragged tail
    (2, 129, 257, 5, 128, False),
    (1, 64, 64, 1, 64, True),          # fewer items than work-groups
    (4, 2048, 2048, 16, 128, True),    # two full rounds of the deal (the second reversed)
    (3, 2048, 2048, 16, 128, True),    # 768 items: a partial reversed round
    (1, 4096, 4096, 20, 128, True),    # 640 items, 20 pairs (not a multiple of 8)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_N{}_Nk{}_H{}_d{}_{}".format(
    *c[:5], "causal" if c[5] else "full"))
def test_persistent_equals_fa_fwd(case):
    gu.need_gpu()
    B, N, Nk, H, d, causal = case
    gu.announce(f"persistent fwd {case}")
    x = wl.make_dense(B, N, H, d, seed=4000 + N + H, Nk=Nk, with_dout=False)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    scale = d ** -0.5
    o1, l1 = fa355.attention_forward(q, k, v, scale, causal)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    fa355.fa_fwd_persistent(q, k, v, o2, l2, scale, causal)
    torch.cuda.synchronize()
    if not gu.fwd_is_key_split(B, H, N, causal):
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
    if B * N * Nk * H <= 2 * 300 * 300 * 8 or gu.fwd_is_key_split(B, H, N, causal):
        o_ref, l_ref = oracle.attention_forward(x["q"], x["k"], x["v"], scale, causal)
        gu.check_forward(o2, l2, o_ref, l_ref, f"persistent {case}")
