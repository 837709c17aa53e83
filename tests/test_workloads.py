"""Seeded input generation (CPU only)."""

import torch

from io_aware_exact_attention_amd import workloads as wl


def test_dense_is_seeded_and_bf16():
    a = wl.make_dense(1, 16, 2, 8, seed=3)
    b = wl.make_dense(1, 16, 2, 8, seed=3)
    for key in ("q", "k", "v", "dout"):
        assert a[key].dtype == torch.bfloat16
        assert torch.equal(a[key], b[key])
    assert not torch.equal(a["q"], a["k"])


def test_k_scale_is_applied_before_rounding():
    g = torch.Generator().manual_seed(9)
    torch.randn((1, 8, 1, 4), generator=g)          # q
    raw_k = torch.randn((1, 8, 1, 4), generator=g)
    x = wl.make_dense(1, 8, 1, 4, seed=9, k_scale=3.0)
    assert torch.equal(x["k"], (raw_k * 3.0).to(torch.bfloat16))


def test_varlen_lengths_and_offsets():
    w = wl.WORKLOADS["varlen_h32_d128_64seq"]
    lens = wl.seq_lengths(w.nseq, w.min_len, w.max_len, w.seed)
    assert len(lens) == 64 and min(lens) >= 128 and max(lens) <= 8192
    cu = wl.cu_seqlens_from_lengths(lens)
    assert cu.dtype == torch.int32 and cu[0] == 0 and int(cu[-1]) == sum(lens)
    assert all(int(cu[i + 1]) - int(cu[i]) == lens[i] for i in range(64))
    small = wl.make_packed([3, 0, 5], 2, 8, seed=1)
    assert small["q"].shape == (8, 2, 8) and small["max_seqlen"] == 5
    assert small["cu_seqlens"].tolist() == [0, 3, 3, 8]


def test_workload_table():
    assert set(wl.WORKLOADS) >= {wl.HEADLINE}
    h = wl.WORKLOADS[wl.HEADLINE]
    assert (h.B, h.H, h.N, h.d, h.causal) == (8, 16, 4096, 128, (True,))
