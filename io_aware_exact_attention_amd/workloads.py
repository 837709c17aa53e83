"""Seeded synthetic workloads: shapes, seeds and input generation.

This module draws the random inputs that both the HIP path and the CPU oracle
consume.  It holds none of the attention arithmetic; it only produces bf16
tensors (and, for packed variable-length batches, cu_seqlens offsets).

Recipe (identical for every consumer):
  * a CPU ``torch.Generator`` seeded with the workload's seed;
  * draws in the order q, k, v, dout, each fp32 N(0, 1) of the full shape;
  * one round-to-nearest-even conversion to bf16 (k is multiplied by
    ``k_scale`` in fp32 before that single rounding, for peaky rows);
  * packed batches: sequence lengths drawn first, from numpy's
    ``default_rng(seed)``, uniform integers in [min_len, max_len] inclusive;
  * decoding workloads draw q, k, v only (k and v have the key/value heads);
  * the FP8 path's random signs (the diagonal of its Hadamard rotation) come
    from their own generator seeded with ``signs_seed``: integers in {0, 1}
    mapped to -1, +1, as fp32.

Dense tensors are [B, N, H, d]; packed tensors are [total, H, d].
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int
    d: int
    causal: tuple
    seed: int
    B: int = 0
    N: int = 0
    k_scale: float = 1.0
    nseq: int = 0
    min_len: int = 0
    max_len: int = 0
    note: str = ""

    @property
    def varlen(self) -> bool:
        return self.nseq > 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The five workloads of the method's evaluation.  Seeds are fixed here once.
WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny", B=1, H=1, N=256, d=64, causal=(False,), seed=1001,
                 note="B1 H1 N256 d64, non-causal"),
        Workload("b4_h16_n1024_d64", B=4, H=16, N=1024, d=64, causal=(False, True), seed=1002,
                 note="B4 H16 N1024 d64, causal and non-causal"),
        Workload("b8_h16_n4096_d128_causal", B=8, H=16, N=4096, d=128, causal=(True,), seed=1003,
                 note="B8 H16 N4096 d128 causal (headline)"),
        Workload("b1_h16_n32768_d128_k3_causal", B=1, H=16, N=32768, d=128, causal=(True,),
                 seed=1004, k_scale=3.0,
                 note="B1 H16 N32768 d128 causal, K scaled by 3 (peaky rows)"),
        Workload("varlen_h32_d128_64seq", H=32, d=128, causal=(True,), seed=1005,
                 nseq=64, min_len=128, max_len=8192,
                 note="64 packed sequences, lengths U[128, 8192], causal per sequence"),
    )
}

HEADLINE = "b8_h16_n4096_d128_causal"


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """Decoding: Nq new query tokens per sequence against an Nk-token key/value
    cache, Hq query heads sharing Hkv key/value heads (grouped-query)."""
    name: str
    B: int
    Nq: int
    Nk: int
    Hq: int
    Hkv: int
    d: int
    causal: bool
    seed: int
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


DECODE_WORKLOADS = {
    w.name: w
    for w in (
        DecodeWorkload("decode_b2_hq32_hkv4_nq4_nk131072_d128", B=2, Nq=4, Nk=131072, Hq=32, Hkv=4,
                       d=128, causal=True, seed=1006,
                       note="4 new tokens against a 128k-token cache, 8 query heads per KV head"),
    )
}


@dataclasses.dataclass(frozen=True)
class Fp8Workload:
    """The FP8 forward on a dense workload's inputs, with the rotation's signs."""
    name: str
    base: str            # the dense workload whose q, k, v are used
    signs_seed: int
    note: str = ""


FP8_WORKLOADS = {
    w.name: w
    for w in (
        Fp8Workload("fp8_b8_h16_n4096_d128_causal", base="b8_h16_n4096_d128_causal", signs_seed=1007,
                    note="FP8 forward on the B8 H16 N4096 d128 causal inputs"),
    )
}


def make_signs(d: int, seed: int) -> torch.Tensor:
    """fp32 [d] of +1 / -1 from a generator of its own."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randint(0, 2, (d,), generator=g).to(torch.float32) * 2 - 1


def seq_lengths(nseq: int, min_len: int, max_len: int, seed: int) -> list[int]:
    """Sequence lengths, uniform integers in [min_len, max_len] inclusive."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(min_len, max_len + 1, size=nseq)]


def cu_seqlens_from_lengths(lengths) -> torch.Tensor:
    """int32 exclusive prefix sum [0, L1, L1+L2, ..., sum L]."""
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return torch.tensor(out, dtype=torch.int32)


def _draw(gen: torch.Generator, shape, mult: float = 1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if mult != 1.0:
        x.mul_(mult)
    return x.to(torch.bfloat16)


def make_dense(B: int, N: int, H: int, d: int, seed: int, k_scale: float = 1.0,
               Nk: Optional[int] = None, with_dout: bool = True) -> dict:
    """bf16 q [B,N,H,d], k/v [B,Nk,H,d], dout [B,N,H,d] from one seeded stream."""
    nk = N if Nk is None else Nk
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    out = {
        "q": _draw(g, (B, N, H, d)),
        "k": _draw(g, (B, nk, H, d), k_scale),
        "v": _draw(g, (B, nk, H, d)),
    }
    if with_dout:
        out["dout"] = _draw(g, (B, N, H, d))
    return out


def make_packed(lengths, H: int, d: int, seed: int, with_dout: bool = True) -> dict:
    """bf16 packed q/k/v/dout [total, H, d] plus cu_seqlens and max_seqlen."""
    lengths = [int(x) for x in lengths]
    total = sum(lengths)
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    out = {
        "q": _draw(g, (total, H, d)),
        "k": _draw(g, (total, H, d)),
        "v": _draw(g, (total, H, d)),
        "cu_seqlens": cu_seqlens_from_lengths(lengths),
        "max_seqlen": max(lengths) if lengths else 0,
        "lengths": lengths,
    }
    if with_dout:
        out["dout"] = _draw(g, (total, H, d))
    return out


def make_decode(B: int, Nq: int, Nk: int, Hq: int, Hkv: int, d: int, seed: int) -> dict:
    """bf16 q [B,Nq,Hq,d], k/v [B,Nk,Hkv,d] from one seeded stream (draws q, k, v)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return {"q": _draw(g, (B, Nq, Hq, d)), "k": _draw(g, (B, Nk, Hkv, d)),
            "v": _draw(g, (B, Nk, Hkv, d))}


def make_inputs(name: str, with_dout: bool = True) -> dict:
    """Inputs of a named workload (CPU, bf16)."""
    if name in FP8_WORKLOADS:
        w8 = FP8_WORKLOADS[name]
        out = make_inputs(w8.base, with_dout=False)
        out["signs"] = make_signs(out["q"].shape[-1], w8.signs_seed)
        return out
    if name in DECODE_WORKLOADS:
        w = DECODE_WORKLOADS[name]
        return make_decode(w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.seed)
    w = WORKLOADS[name]
    if w.varlen:
        lens = seq_lengths(w.nseq, w.min_len, w.max_len, w.seed)
        return make_packed(lens, w.H, w.d, w.seed, with_dout)
    return make_dense(w.B, w.N, w.H, w.d, w.seed, w.k_scale, with_dout=with_dout)
