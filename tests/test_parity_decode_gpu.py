"""Split-KV decoding with grouped-query heads on the GPU against the oracle.

Same bars as the other forward tests: O max-abs <= 1e-2, LSE max-abs <= 1e-3.
Cases cover packed-row counts below, at and above one 32-row tile, one token,
Nq = Nk, key counts that leave a ragged last tile and fewer keys than one tile,
both masks and both head dims; the decoding workload runs at full size and is
compared on whole sampled (sequence, key/value head) groups.
"""

import pytest
import torch

import oracle
from io_aware_exact_attention_amd import fa355, workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    # B, Nq, Nk, Hq, Hkv, d, causal
    (2, 4, 1000, 16, 2, 128, True),     # 8 heads x 4 tokens = one full tile
    (2, 4, 1000, 16, 2, 128, False),
    (1, 1, 77, 4, 4, 64, True),         # one token, no grouping, ragged keys
    (2, 3, 4099, 16, 2, 128, True),     # 24 packed rows: padded tile
    (1, 4, 300, 32, 2, 64, True),       # 64 packed rows: two tiles
    (1, 2, 5, 2, 1, 128, True),         # fewer keys than one tile
    (1, 1, 1, 8, 1, 128, False),        # a single key
    (1, 8, 8, 4, 2, 64, True),          # Nq = Nk: the ordinary causal mask
]


def _run(B, Nq, Nk, Hq, Hkv, d, causal, seed):
    gu.need_gpu()
    gu.announce(f"decode B{B} Nq{Nq} Nk{Nk} Hq{Hq} Hkv{Hkv} d{d} causal={causal}")
    x = wl.make_decode(B, Nq, Nk, Hq, Hkv, d, seed)
    dev = torch.device("cuda", 0)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    scale = d ** -0.5
    o, lse = fa355.attention_decode(q, k, v, scale, causal)
    torch.cuda.synchronize()
    return x, o, lse, scale


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Nq{}_Nk{}_Hq{}_Hkv{}_d{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
def test_decode_small(case):
    x, o, lse, scale = _run(*case, seed=2000 + sum(case[:6]))
    o_ref, lse_ref = oracle.decode_forward(x["q"], x["k"], x["v"], scale, case[6])
    gu.check_forward(o, lse, o_ref, lse_ref, f"decode {case}")


def test_decode_deterministic():
    a = _run(2, 4, 3000, 16, 2, 128, True, seed=7)
    b = _run(2, 4, 3000, 16, 2, 128, True, seed=7)
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


def test_decode_workload_full_size():
    w = wl.DECODE_WORKLOADS["decode_b2_hq32_hkv4_nq4_nk131072_d128"]
    x, o, lse, scale = _run(w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.causal, seed=w.seed)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    G = w.Hq // w.Hkv
    for b, hkv in ((0, 0), (1, 3)):
        hs = slice(hkv * G, (hkv + 1) * G)
        xs = {"q": x["q"][b:b + 1, :, hs].contiguous(),
              "k": x["k"][b:b + 1, :, hkv:hkv + 1].contiguous(),
              "v": x["v"][b:b + 1, :, hkv:hkv + 1].contiguous()}
        o_ref, lse_ref = oracle.decode_forward(xs["q"], xs["k"], xs["v"], scale, w.causal)
        gu.check_forward(o[b:b + 1, :, hs], lse[b:b + 1, hs], o_ref, lse_ref,
                         f"decode workload b={b} kv head {hkv}")


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_cache_rows_past_a_sequence_read_as_zeros(causal):
    """The last key chunk of sequence 0 runs past its 700 cached rows into sequence
    1's cache, which here is all NaN: those rows must read as zeros."""
    gu.need_gpu()
    gu.announce(f"decode NaN neighbours causal={causal}")
    dev = torch.device("cuda", 0)
    scale = 128 ** -0.5
    y = wl.make_decode(2, 4, 700, 8, 2, 128, seed=2100)
    yn = {n: t.clone() for n, t in y.items()}
    for t in yn.values():
        t[1] = float("nan")
    o, lse = fa355.attention_decode(*(yn[n].to(dev) for n in ("q", "k", "v")), scale, causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_forward(y["q"][:1], y["k"][:1], y["v"][:1], scale, causal)
    gu.check_forward(o[:1], lse[:1].cpu(), o_ref, lse_ref, "decode sequence 0")
