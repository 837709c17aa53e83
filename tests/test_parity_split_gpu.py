"""The key-split forward on the GPU against the oracle.

fa_fwd runs causal grids with at most one 128-row query tile per CU (or two,
for sequences of at least 16 such tiles) on the key-split kernel: one 8-wave
work-group per query tile, whose two halves of waves take the first ceil(n/2)
and the last floor(n/2) of the tile's n key tiles and merge their
online-softmax states through LDS.  The cases cover one
key tile (an empty second half), odd and even tile counts, ragged query and key
tails, both head dims, and the largest grid that takes this path (two query
tiles per CU).  Outputs are pre-filled with NaN so that a row no wave writes
fails; each is then compared element by element with the oracle, and the
backward is run on the kernel's LSE.
"""

import pytest
import torch

from io_aware_exact_attention_amd import fa355, workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    # B, N, H, d
    (1, 1, 1, 64),
    (1, 33, 2, 128),
    (1, 64, 1, 64),
    (1, 65, 3, 128),       # two key tiles in the last query tile: one per half
    (2, 127, 2, 64),
    (1, 128, 1, 128),
    (1, 129, 2, 64),       # ragged second query tile with one row
    (1, 192, 1, 128),      # three key tiles: 2 + 1
    (2, 255, 3, 64),
    (1, 257, 5, 128),
    (1, 500, 2, 64),
    (1, 1000, 4, 128),
    (3, 1024, 5, 64),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_N{}_H{}_d{}".format(*c))
def test_key_split_forward(case):
    gu.need_gpu()
    B, N, H, d = case
    assert gu.fwd_is_key_split(B, H, N, True)
    gu.announce(f"key-split fwd {case}")
    x = wl.make_dense(B, N, H, d, seed=7100 + 3 * N + H + d)
    scale = d ** -0.5
    dev = torch.device("cuda", 0)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    fa355.fa_fwd(q, k, v, o, lse, scale, True)
    grads = fa355.attention_backward(q, k, v, o, do, lse, scale, True)
    torch.cuda.synchronize()
    r = gu.oracle_dense(x, scale, True)
    assert torch.isfinite(lse).all(), "an LSE row was not written"
    gu.check_forward(o, lse, r["o"], r["lse"], f"key-split {case}")
    gu.check_grads(grads, r["grads"], f"key-split {case}")


def test_key_split_largest_grid():
    """512 query tiles of N = 4096 on the 256-CU MI355X (B1 H16 N4096 d128): the
    largest grid the key-split kernel takes; three heads compared in full."""
    gu.need_gpu()
    B, N, H, d = 1, 4096, 16, 128
    if not gu.fwd_is_key_split(B, H, N, True):
        pytest.skip("this device has fewer work-group slots than 512 query tiles")
    gu.announce("key-split fwd largest grid")
    x = wl.make_dense(B, N, H, d, seed=7300, with_dout=False)
    scale = d ** -0.5
    dev = torch.device("cuda", 0)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    fa355.fa_fwd(q, k, v, o, lse, scale, True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    import oracle
    for h in (0, 7, 15):
        sl = lambda t: t[:, :, h:h + 1]
        o_ref, l_ref = oracle.attention_forward(sl(x["q"]), sl(x["k"]), sl(x["v"]), scale, True)
        gu.check_forward(sl(o), lse[:, h:h + 1], o_ref, l_ref, f"key-split h{h}")
