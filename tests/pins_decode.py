"""Checks that tie the decoding oracle (oracle/decode.py) to facts outside it.

Each ``pin_*`` takes a module with decode_forward, decode_split_partials and
merge_splits (normally ``oracle``; the mutation tests pass copies of
oracle/decode.py with a planted mistake).  The facts:

* grouped-query decoding is ordinary attention per query head against its
  key/value head ("LLM Systems 22: Flash Attention", §5.2, GQA packing), so it
  must equal the dense oracle (pinned on its own) run on key/value heads
  repeated per group, and torch-CPU float64 ``scaled_dot_product_attention``
  with an explicit mask;
* splitting the keys into chunks and merging the chunk statistics gives the
  one-shot result ("LLM Systems 22: Flash Attention", §5.2 Split-KV), for any
  split, and the merge is associative.
"""

from __future__ import annotations

import torch
import torch.nn.functional as F

import oracle as dense


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64) * scale


def _expand(kv, G):
    """[B, Nk, Hkv, d] -> [B, Nk, Hkv*G, d] with query head h on key/value head h // G."""
    return kv.repeat_interleave(G, dim=2)


def pin_dense_equivalence(orc):
    # Nq == Nk: decoding is dense attention on the expanded heads (both masks)
    q = _rand((2, 23, 6, 16), 301)
    k, v = _rand((2, 23, 2, 16), 302), _rand((2, 23, 2, 16), 303)
    for causal in (False, True):
        o, lse = orc.decode_forward(q, k, v, 0.3, causal)
        o_ref, lse_ref = dense.attention_forward(q, _expand(k, 3), _expand(v, 3), 0.3, causal)
        assert (o - o_ref).abs().max().item() < 1e-12, causal
        assert (lse - lse_ref).abs().max().item() < 1e-12, causal


def pin_sdpa_bottom_right(orc):
    # Nq < Nk: query i sees keys j <= i + Nk - Nq; compare with SDPA + explicit mask
    B, Nq, Nk, Hq, Hkv, d, scale = 2, 4, 37, 8, 2, 16, 0.25
    q = _rand((B, Nq, Hq, d), 311, 2.0)
    k, v = _rand((B, Nk, Hkv, d), 312), _rand((B, Nk, Hkv, d), 313)
    G = Hq // Hkv
    ke, ve = _expand(k, G), _expand(v, G)
    for causal in (False, True):
        o, lse = orc.decode_forward(q, k, v, scale, causal)
        mask = torch.ones(Nq, Nk, dtype=torch.bool)
        if causal:
            mask = torch.arange(Nk)[None, :] <= torch.arange(Nq)[:, None] + (Nk - Nq)
        o_ref = F.scaled_dot_product_attention(q.transpose(1, 2), ke.transpose(1, 2),
                                               ve.transpose(1, 2), attn_mask=mask,
                                               scale=scale).transpose(1, 2)
        s = scale * torch.einsum("bihd,bjhd->bhij", q, ke)
        lse_ref = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
        assert (o - o_ref).abs().max().item() < 1e-12, causal
        assert (lse - lse_ref).abs().max().item() < 1e-12, causal


def pin_single_token(orc):
    # one query token is the newest position: the causal mask hides nothing
    q = _rand((3, 1, 4, 8), 321)
    k, v = _rand((3, 19, 1, 8), 322), _rand((3, 19, 1, 8), 323)
    o1, l1 = orc.decode_forward(q, k, v, 0.5, True)
    o0, l0 = orc.decode_forward(q, k, v, 0.5, False)
    assert (o1 - o0).abs().max().item() == 0 and (l1 - l0).abs().max().item() == 0
    # and it is the dense oracle on the expanded heads
    o_ref, l_ref = dense.attention_forward(q, _expand(k, 4), _expand(v, 4), 0.5, False)
    assert (o1 - o_ref).abs().max().item() < 1e-12 and (l1 - l_ref).abs().max().item() < 1e-12


def pin_split_merge(orc):
    B, Nq, Nk, Hq, Hkv, d = 2, 3, 50, 4, 2, 8
    q = _rand((B, Nq, Hq, d), 331, 3.0)
    k, v = _rand((B, Nk, Hkv, d), 332), _rand((B, Nk, Hkv, d), 333)
    splits = ([0, 50], [0, 1, 50], [0, 17, 18, 40, 48, 49, 50], list(range(51)), [0, 25, 49, 50])
    for causal in (False, True):
        o_ref, lse_ref = orc.decode_forward(q, k, v, 0.4, causal)
        for bnd in splits:
            o, lse = orc.merge_splits(orc.decode_split_partials(q, k, v, 0.4, causal, bnd))
            assert (o - o_ref).abs().max().item() < 1e-12, (causal, bnd)
            assert (lse - lse_ref).abs().max().item() < 1e-12, (causal, bnd)
        # the last chunk [49, 50) is invisible to the first rows under the causal mask
        parts = orc.decode_split_partials(q, k, v, 0.4, True, [0, 48, 49, 50])
        assert torch.isinf(parts[2][1][:, :, 0]).all() and (parts[2][0][:, 0] == 0).all()
    # associativity: merging a merge with a chunk equals merging the three chunks
    p3 = orc.decode_split_partials(q, k, v, 0.4, False, [0, 11, 30, 50])
    left = orc.merge_splits([orc.merge_splits(p3[:2]), p3[2]])
    right = orc.merge_splits([p3[0], orc.merge_splits(p3[1:])])
    flat = orc.merge_splits(p3)
    for a in (left, right):
        assert (a[0] - flat[0]).abs().max().item() < 1e-13
        assert (a[1] - flat[1]).abs().max().item() < 1e-13


ALL_PINS = [pin_dense_equivalence, pin_sdpa_bottom_right, pin_single_token, pin_split_merge]
