"""Decoding attention with grouped-query heads and split keys, float64 on the CPU.

TEST INFRASTRUCTURE (see the package docstring): only the tests, the smoke
check and the CPU-baseline leg of the benchmark use this module.

Sources (page title, then the section on that page):

* The decoding regime -- one to a few query tokens against a long key/value
  cache -- and its remedy, split-KV ("Flash-Decoding"): the keys are cut into
  independent chunks, each chunk yields a partial output with its own
  normalisation statistics (m, l), and a light reduction merges the chunks:
  "LLM Systems 22: Flash Attention", §5.1 Motivation and §5.2 Solution.
* Grouped-query attention: several query heads share one key/value head, and
  those query heads' rows are packed together onto the matrix unit: same page,
  §5.2 (GQA Packing).
* Each head's attention is the definition O = softmax(scale * Q K^T) V with the
  safe (max-subtracted) softmax and LSE = m + ln(l) per query row:
  "08 · FlashAttention", §一 and §二; "LLM Systems 22: Flash Attention", §3.2.

Readings taken where the pages are silent:

* Head mapping: with Hq query heads and Hkv key/value heads (G = Hq / Hkv),
  query head h reads key/value head h // G (consecutive query heads share).
* Causal alignment: the Nq query tokens are the last Nq positions of the
  sequence whose keys are cached, so query i sees key j iff j <= i + (Nk - Nq).
  (For Nq = Nk this is the ordinary causal mask; for Nq = 1 every key.)
* A split with no visible key for a row contributes LSE_s = -inf and O_s = 0.

Layout: q [B, Nq, Hq, d]; k, v [B, Nk, Hkv, d]; O [B, Nq, Hq, d]; LSE [B, Hq, Nq].
"""

from __future__ import annotations

from typing import Sequence

import torch

_NEG_INF = float("-inf")


def _f64(x: torch.Tensor) -> torch.Tensor:
    return x.detach().to(device="cpu", dtype=torch.float64)


def _check(q, k, v, causal):
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q [B, Nq, Hq, d]; k, v [B, Nk, Hkv, d]")
    B, Nq, Hq, d = q.shape
    if k.shape[0] != B or k.shape[3] != d or Hq % k.shape[2] != 0:
        raise ValueError("batch and head dim must agree and Hkv must divide Hq")
    if causal and Nq > k.shape[1]:
        raise ValueError("causal decoding needs Nq <= Nk")
    return B, Nq, Hq, d, k.shape[1], k.shape[2]


def _head_scores(qh, kh, scale, causal, key0, nq, nk):
    """scale * q k^T for one head, keys key0.. of the cache; invisible -> -inf.

    qh: [Nq, d]; kh: [K, d]; returns [Nq, K].
    """
    s = scale * torch.matmul(qh, kh.transpose(0, 1))
    if causal:
        qi = torch.arange(nq).unsqueeze(1)
        kj = torch.arange(key0, key0 + kh.shape[0]).unsqueeze(0)
        s = s.masked_fill(kj > qi + (nk - nq), _NEG_INF)
    return s


def decode_forward(q, k, v, scale: float, causal: bool):
    """O and LSE of every query head against its key/value head, in one shot."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Nq, Hq, d, Nk, Hkv = _check(q, k, v, causal)
    G = Hq // Hkv
    o = torch.empty(B, Nq, Hq, d, dtype=torch.float64)
    lse = torch.empty(B, Hq, Nq, dtype=torch.float64)
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            s = _head_scores(q[b, :, h], k[b, :, kv], scale, causal, 0, Nq, Nk)
            m = s.amax(dim=-1, keepdim=True)
            e = torch.exp(s - m)
            l = e.sum(dim=-1, keepdim=True)
            o[b, :, h] = torch.matmul(e / l, v[b, :, kv])
            lse[b, h] = (m + torch.log(l)).squeeze(-1)
    return o, lse


def decode_split_partials(q, k, v, scale: float, causal: bool, boundaries: Sequence[int]):
    """Per key chunk [b_s, b_{s+1}): the chunk's own normalised output and LSE.

    Returns a list of (O_s [B, Nq, Hq, d], LSE_s [B, Hq, Nq]); rows that see no
    key of the chunk get O_s = 0 and LSE_s = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Nq, Hq, d, Nk, Hkv = _check(q, k, v, causal)
    G = Hq // Hkv
    bnd = [int(x) for x in boundaries]
    if bnd[0] != 0 or bnd[-1] != Nk or any(b1 <= b0 for b0, b1 in zip(bnd, bnd[1:])):
        raise ValueError("boundaries must rise strictly from 0 to Nk")
    out = []
    for j0, j1 in zip(bnd, bnd[1:]):
        o_s = torch.zeros(B, Nq, Hq, d, dtype=torch.float64)
        lse_s = torch.full((B, Hq, Nq), _NEG_INF, dtype=torch.float64)
        for b in range(B):
            for h in range(Hq):
                kv = h // G
                s = _head_scores(q[b, :, h], k[b, j0:j1, kv], scale, causal, j0, Nq, Nk)
                m = s.amax(dim=-1, keepdim=True)
                live = (m > _NEG_INF).squeeze(-1)
                if not live.any():
                    continue
                e = torch.exp(s[live] - m[live])
                l = e.sum(dim=-1, keepdim=True)
                o_s[b, live, h] = torch.matmul(e / l, v[b, j0:j1, kv])
                lse_s[b, h, live] = (m[live] + torch.log(l)).squeeze(-1)
        out.append((o_s, lse_s))
    return out


def merge_splits(partials):
    """Combine chunk results: LSE = ln sum_s e^(LSE_s), O = sum_s e^(LSE_s - LSE) O_s.

    This is the online-softmax merge of (m, l, O) statistics ("08 · FlashAttention",
    §二) written with each chunk's normalised output: e^(LSE_s) = e^(m_s) l_s.
    """
    lses = torch.stack([p[1] for p in partials])          # [S, B, Hq, Nq]
    top = lses.amax(dim=0)
    safe = torch.where(top > _NEG_INF, top, torch.zeros_like(top))
    w = torch.exp(lses - safe)                            # -inf chunks -> 0
    tot = w.sum(dim=0)
    lse = safe + torch.log(tot)
    o = torch.zeros_like(partials[0][0])
    for (o_s, _), w_s in zip(partials, w):
        o += (w_s / tot).permute(0, 2, 1).unsqueeze(-1) * o_s
    return o, lse
