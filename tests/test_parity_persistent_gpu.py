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


CARRY_CASES = [
    # B, N, H: causal d = 128 grids of several rounds with at most 32 tiles per
    # sequence, which fa_fwd runs on the persistent kernel with carried items
    (4, 2048, 16),    # two rounds
    (8, 4096, 16),    # the headline shape: eight rounds
    (3, 4000, 16),    # ragged tail, three rounds
    (5, 2500, 13),    # ragged, 65 pairs (not a multiple of 8)
]


@pytest.mark.parametrize("case", CARRY_CASES, ids=lambda c: "B{}_N{}_H{}".format(*c))
def test_carried_items_equal_per_tile_kernel(case):
    """The persistent forward's carried items (each item issues its successor's
    first K/V tiles and Q rows before its own stores) compute each tile exactly
    as the per-tile kernel does, which the varlen entry point always runs: on
    equal-length sequences, packed, O and LSE must be equal bit for bit; two
    sampled (batch, head) slices are also compared with the oracle."""
    gu.need_gpu()
    B, N, H = case
    d = 128
    if gu.fwd_is_key_split(B, H, N, True):
        pytest.skip("this device runs the key-split kernel for this grid")
    gu.announce(f"carried forward {case}")
    x = wl.make_dense(B, N, H, d, seed=4500 + N + H, with_dout=False)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    scale = d ** -0.5
    o1, l1 = fa355.attention_forward(q, k, v, scale, True)
    cu = (torch.arange(B + 1, dtype=torch.int32) * N).cuda()
    pk = lambda t: t.reshape(B * N, H, d)
    o2, l2 = fa355.attention_forward_varlen(pk(q), pk(k), pk(v), cu, cu, N, N, scale, True)
    torch.cuda.synchronize()
    assert torch.equal(pk(o1), o2) and torch.equal(l1, l2)
    for b, h in ((0, 0), (B - 1, H - 1)):
        xs = {n: x[n][b:b + 1, :, h:h + 1] for n in ("q", "k", "v")}
        o_ref, l_ref = oracle.attention_forward(xs["q"], xs["k"], xs["v"], scale, True)
        gu.check_forward(o1[b:b + 1, :, h:h + 1], l1[b:b + 1, h:h + 1], o_ref, l_ref, f"carried {case} b{b} h{h}")
