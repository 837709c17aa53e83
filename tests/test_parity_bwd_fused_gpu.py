"""The one-launch backward of small dense grids on the GPU.

fa_bwd runs grids of at most 6 (causal) or 2 (non-causal) dK/dV plus dQ work
items per CU as the row-dot kernel followed by one launch that holds both passes'
work items.  Each work
item is the same computation as in the two-kernel backward (the row-dot kernel
stores the same -D and LSE * log2(e) bit for bit as the dQ kernel's folded
row-dot), so the gradients must equal the stage entry points' (fa_bwd_dq_dot,
then fa_bwd_dkdv) bit for bit; they are also compared with the oracle.  Cases
cover both masks, Nq != Nk in both directions (more dQ than dK/dV items and the
reverse), ragged tails, head and batch counts that are not multiples of 8, and
the largest grids that take this path on a 256-CU MI355X (causal B6 H16 N1024,
non-causal B2 H16 N1024).
"""

import pytest
import torch

from io_aware_exact_attention_amd import fa355, workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    # B, Nq, Nk, H, d, causal
    (1, 1, 1, 1, 64, True),
    (2, 200, 200, 3, 128, True),
    (1, 300, 129, 5, 64, False),     # 3 dQ tiles, 2 dK/dV tiles per pair
    (3, 100, 513, 2, 128, False),    # 1 dQ tile, 5 dK/dV tiles per pair
    (2, 1000, 1000, 7, 64, True),
    (1, 2048, 2048, 8, 128, True),
    (2, 1024, 1024, 16, 64, False),  # the largest non-causal grid on this path
    (4, 1024, 1024, 16, 64, True),
    (6, 1024, 1024, 16, 64, True),   # the largest causal grid on this path
]


def _ids(c):
    return "B{}_Nq{}_Nk{}_H{}_d{}_{}".format(*c[:5], "causal" if c[5] else "full")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_fused_backward(case):
    gu.need_gpu()
    B, Nq, Nk, H, d, causal = case
    if not gu.bwd_is_fused(B, H, Nq, Nk, causal):
        pytest.skip("this device takes the two-kernel backward for this grid")
    gu.announce(f"fused bwd {case}")
    x = wl.make_dense(B, Nq, H, d, seed=7500 + Nq + 3 * Nk + H + d, Nk=Nk)
    scale = d ** -0.5
    dev = torch.device("cuda", 0)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    o, lse = fa355.attention_forward(q, k, v, scale, causal)
    nws = fa355.fa_bwd_workspace_bytes(B, H, Nq, d) // 4
    ws1, ws2 = (torch.full((nws,), float("nan"), device=dev) for _ in range(2))
    g1 = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    g2 = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    fa355.fa_bwd(q, k, v, o, do, lse, g1[0], g1[1], g1[2], ws1, scale, causal)
    fa355.fa_bwd_dq_dot(q, k, v, o, do, lse, ws2, g2[0], scale, causal)
    fa355.fa_bwd_dkdv(q, k, v, do, ws2, g2[1], g2[2], scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(ws1, ws2), "workspace differs from the dQ kernel's folded row-dot"
    for name, a, b in zip(("dq", "dk", "dv"), g1, g2):
        assert torch.equal(a, b), f"{name} differs from the two-kernel backward"
    if B * Nq * Nk * H <= 4 * 1024 * 1024:
        r = gu.oracle_dense(x, scale, causal)
        gu.check_grads(g1, r["grads"], f"fused {case}")
