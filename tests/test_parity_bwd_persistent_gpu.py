"""The persistent backward grids on the GPU.

For dense causal backwards that do not take the one-launch form, a pass
(dK/dV over 128-key tiles, dQ over 128-row tiles) with more than two work items
per CU and either at most eight per CU or at most 32 tiles per sequence runs on
a persistent grid of two work-groups per CU that deals the items in the
per-tile grid's order.  Each item is the same
arithmetic as in the per-tile kernels, which the varlen entry point always
runs; on equal-length sequences, packed, with the dense forward's O and LSE,
it must give the same gradients bit for bit.  Sampled (batch entry, head)
pairs are also compared with the oracle.  Cases: the headline shape (eight
rounds), the largest and smallest grids of the four-round range at d = 128 and
d = 64 on a 256-CU MI355X, and ragged ones (N not a multiple of 128, head and
batch counts not multiples of 8, three rounds of the grid).
"""

import pytest
import torch

import oracle
from io_aware_exact_attention_amd import fa355, workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    # B, N, H, d
    (8, 4096, 16, 128),   # the headline shape: 4096 items per pass, eight rounds
    (8, 2048, 16, 128),   # 2048 items per pass: four rounds
    (4, 4096, 16, 128),
    (5, 2500, 13, 128),   # 1300 items per pass, ragged
    (8, 2048, 16, 64),
    (6, 2900, 11, 64),    # 1518 items per pass, ragged
]


def _ids(c):
    return "B{}_N{}_H{}_d{}".format(*c)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_persistent_backward(case):
    gu.need_gpu()
    B, N, H, d = case
    if not any(gu.bwd_is_persistent(B, H, N, N, True)):
        pytest.skip("this device takes per-tile grids for this backward")
    gu.announce(f"persistent bwd {case}")
    x = wl.make_dense(B, N, H, d, seed=8100 + N + H + d)
    scale = d ** -0.5
    dev = torch.device("cuda", 0)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    o, lse = fa355.attention_forward(q, k, v, scale, True)
    g = fa355.attention_backward(q, k, v, o, do, lse, scale, True)
    cu = (torch.arange(B + 1, dtype=torch.int32) * N).to(dev)
    pk = lambda t: t.reshape(B * N, H, d)
    gv = fa355.attention_backward_varlen(pk(q), pk(k), pk(v), pk(o), pk(do), lse, cu, cu, N, N, scale, True)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), g, gv):
        assert torch.equal(pk(a), b), f"{name} differs from the per-tile kernels"
    for b, h in ((0, 0), (B - 1, H - 1)):
        xs = {n: x[n][b:b + 1, :, h:h + 1] for n in ("q", "k", "v", "dout")}
        r = oracle.attention_backward(xs["q"], xs["k"], xs["v"], xs["dout"], scale, True)[:3]
        gu.check_grads([t[b:b + 1, :, h:h + 1] for t in g], r, f"persistent {case} b{b} h{h}")
