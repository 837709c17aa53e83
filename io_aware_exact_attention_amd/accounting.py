"""Algorithmic FLOP and byte counts for exact attention (no hardware numbers).

Conventions, stated once:

* ``pairs``: the (query, key) score entries a pass must evaluate: Nq*Nk, or
  N(N+1)/2 when causal (key j visible to query i iff j <= i).
* Forward FLOPs = 4 d pairs: two matrix products, S = Q K^T and O = P V, each
  2 d FLOPs per pair ("08 · FlashAttention", §一 counts 4 n^2 d for the
  forward of one head).
* Backward FLOPs = 10 d pairs: five products, the recomputed S, dV = P^T dO,
  dP = dO V^T, dQ = dS K and dK = dS^T Q.  Recomputing S is the extra work
  that "LLM Systems 22: Flash Attention", §3.3 attributes to the backward.
* Forward bytes (compulsory HBM traffic, bf16 tensors, fp32 LSE): read Q, K,
  V, write O and LSE -> per token and head 2d*4 + 4 = 8d + 4.
* Backward bytes: read Q, K, V, O, dO and LSE, write dQ, dK, dV, and write
  then read the fp32 row vector D = rowsum(dO * O) -> 2d*8 + 4 + 8 = 16d + 12.

The worked IO example of "08 · FlashAttention", §一 (n = 4096, d = 128, bf16,
one head of one sample) is reproduced by ``standard_attention_io``.
"""

from __future__ import annotations

BF16_BYTES = 2
FP32_BYTES = 4


def pairs(nq: int, nk: int, causal: bool) -> int:
    if causal:
        if nq != nk:
            raise ValueError("causal pairs need nq == nk")
        return nq * (nq + 1) // 2
    return nq * nk


def flops_fwd(npairs: int, d: int) -> int:
    return 4 * d * npairs


def flops_bwd(npairs: int, d: int) -> int:
    return 10 * d * npairs


def bytes_fwd(tokens_q: int, tokens_k: int, H: int, d: int) -> int:
    return H * (tokens_q * (2 * d * BF16_BYTES + FP32_BYTES) + tokens_k * 2 * d * BF16_BYTES)


def bytes_bwd(tokens_q: int, tokens_k: int, H: int, d: int) -> int:
    q_side = tokens_q * (4 * d * BF16_BYTES + FP32_BYTES + 2 * FP32_BYTES)  # Q, O, dO, dQ, LSE, D w+r
    k_side = tokens_k * 4 * d * BF16_BYTES                                 # K, V, dK, dV
    return H * (q_side + k_side)


def dense_counts(B: int, H: int, N: int, d: int, causal: bool, Nk: int | None = None) -> dict:
    nk = N if Nk is None else Nk
    p = B * H * pairs(N, nk, causal)
    return {
        "pairs": p,
        "flops_fwd": flops_fwd(p, d),
        "flops_bwd": flops_bwd(p, d),
        "bytes_fwd": bytes_fwd(B * N, B * nk, H, d),
        "bytes_bwd": bytes_bwd(B * N, B * nk, H, d),
    }


def varlen_counts(lengths, H: int, d: int, causal: bool) -> dict:
    p = H * sum(pairs(n, n, causal) for n in lengths)
    tokens = sum(lengths)
    return {
        "pairs": p,
        "flops_fwd": flops_fwd(p, d),
        "flops_bwd": flops_bwd(p, d),
        "bytes_fwd": bytes_fwd(tokens, tokens, H, d),
        "bytes_bwd": bytes_bwd(tokens, tokens, H, d),
    }


def standard_attention_io(n: int, d: int, elem_bytes: int = BF16_BYTES) -> dict:
    """IO of the standard (non-tiled) attention for one head of one sample.

    The score matrix S and the probabilities P are n x n each and make four
    HBM trips (write S, read S, write P, read P); Q, K, V and O are n x d.
    Compute is counted as 4 n^2 d.
    """
    s_bytes = n * n * elem_bytes
    round_trips = 4 * s_bytes
    qkvo = 4 * n * d * elem_bytes
    flops = 4 * n * n * d
    moved = round_trips + qkvo
    return {
        "score_matrix_bytes": s_bytes,
        "score_round_trip_bytes": round_trips,
        "qkvo_bytes": qkvo,
        "intermediate_share": round_trips / moved,
        "flops": flops,
        "bytes_moved": moved,
        "arithmetic_intensity": flops / moved,
    }


def sfu_tile_budget(block_m: int, block_n: int, d: int, mma_flops_per_clk: float,
                    exp_per_clk: float) -> dict:
    """Cycles for one block_m x block_n tile: both products vs its exponentials."""
    mma = 2 * 2 * block_m * block_n * d
    exps = block_m * block_n
    return {
        "mma_flops": mma,
        "mma_cycles": mma / mma_flops_per_clk,
        "exps": exps,
        "exp_cycles": exps / exp_per_clk,
    }
