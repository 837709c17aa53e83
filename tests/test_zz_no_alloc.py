"""fa_bwd_noalloc (the backward that keeps its workspace in a static device array)
against fa_bwd with a caller workspace, through the C ABI: two calls in a row,
the second on a smaller input, each bitwise equal to fa_bwd and within the
gradient tolerance of the CPU oracle."""

import pytest
import torch

from io_aware_exact_attention_amd import fa355
from io_aware_exact_attention_amd import workloads as wl

from tests.gpu_util import announce, check_grads, need_gpu, oracle_dense

pytestmark = pytest.mark.gpu


def _grads_both_ways(x, scale, causal):
    dev = torch.device("cuda", 0)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    o, lse = fa355.attention_forward(q, k, v, scale, causal)
    B, N, H, d = q.shape
    ws = torch.empty(fa355.fa_bwd_workspace_bytes(B, H, N, d) // 4, dtype=torch.float32, device=dev)
    ref = [torch.empty_like(t) for t in (q, k, v)]
    fa355.fa_bwd(q, k, v, o, do, lse, *ref, ws, scale, causal)
    got = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    fa355.fa_bwd_noalloc(q, k, v, o, do, lse, *got, scale, causal)
    torch.cuda.synchronize()
    return [t.cpu() for t in got], [t.cpu() for t in ref]


@pytest.mark.parametrize("causal", [True, False])
def test_noalloc_matches_fa_bwd_twice_smaller_second(causal):
    need_gpu()
    # the second call is smaller, so stale values of the first call's larger
    # planes remain in the shared array beyond what the second one writes
    for (B, N, H, d, seed) in ((2, 777, 3, 128, 4101), (1, 200, 2, 64, 4102)):
        announce(f"fa_bwd_noalloc B{B} N{N} H{H} d{d} causal={causal}")
        x = wl.make_dense(B, N, H, d, seed=seed)
        scale = d ** -0.5
        got, ref = _grads_both_ways(x, scale, causal)
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name} differs from fa_bwd"
        check_grads(got, oracle_dense(x, scale, causal)["grads"], f"noalloc N{N} d{d}")
