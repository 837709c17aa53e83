"""Exact softmax attention in float64 on the CPU: the definition, written out.

TEST INFRASTRUCTURE (see the package docstring): only the tests, the smoke
check and the CPU-baseline leg of the benchmark use this module.

Sources (page title, then the section on that page):

* Definition O = softmax(S) V with S = Q K^T scaled by 1/sqrt(d):
  "08 · FlashAttention", §一 (standard attention); "LLM Systems 22: Flash
  Attention", §2.1 Attention.  The scale is a caller argument here.
* Safe softmax (subtract the row maximum before exponentiating):
  "08 · FlashAttention", §二 (standard softmax formula).
* Saved per-row statistic: one log-sum-exp per query row, LSE = m + ln(l),
  where m is the row maximum and l the denominator: "LLM Systems 22: Flash
  Attention", §3.2 Backward: Recomputation.
* Online softmax update with running max m, running sum l and an
  unnormalised accumulator O, normalised once at the end: "08 · FlashAttention",
  §二 (the m_new, l_new, O_new update).
* Causal masking (key j visible to query i iff j <= i): "08 · FlashAttention",
  §四 (is_causal is the one supported mask).
* Varlen packing with cu_seqlens prefix offsets: "08 · FlashAttention", §四;
  packed [total, heads, head_dim] tensors: "Flash Attention 实现深度解析", §3.1.
* Gradients: the pages only say that the backward recomputes P from the saved
  statistics; the formulas below are the chain rule of the definition
  (dV = P^T dO, dP = dO V^T, dS = P * (dP - D) with D = rowsum(P * dP),
  dQ = scale dS K, dK = scale dS^T Q).

Layout: dense tensors are [B, N, H, d] (token-major, then head, then head
dimension), LSE is [B, H, N].  Every input is upcast exactly to float64 first.

Query rows are evaluated in groups of ``row_chunk`` rows.  Each row of a
softmax depends on that row only, so this is the definition itself; the one
effect on the arithmetic is that dK and dV, which sum over query rows, are
summed group by group (a float64 rounding-order difference only).
"""

from __future__ import annotations

from typing import Sequence

import torch

_NEG_INF = float("-inf")


def _f64(x: torch.Tensor) -> torch.Tensor:
    return x.detach().to(device="cpu", dtype=torch.float64)


def _check_dense(q, k, v, causal):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("dense tensors are [B, N, H, d]")
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[2:] != k.shape[2:]:
        raise ValueError("q [B,Nq,H,d], k and v [B,Nk,H,d] must agree")
    if causal and q.shape[1] != k.shape[1]:
        # Causal alignment for Nq != Nk is not fixed by the pages.
        raise ValueError("causal attention needs Nq == Nk")


def _scores(q_rows: torch.Tensor, keys: torch.Tensor, scale: float,
            row0: int, causal: bool) -> torch.Tensor:
    """S = scale * q k^T for query rows row0.. (per head), causal entries -> -inf.

    q_rows: [H, R, d]; keys: [H, K, d]; returns [H, R, K].
    """
    s = scale * torch.matmul(q_rows, keys.transpose(-1, -2))
    if causal:
        r, kk = s.shape[-2], s.shape[-1]
        qi = torch.arange(row0, row0 + r).unsqueeze(1)
        kj = torch.arange(kk).unsqueeze(0)
        s = s.masked_fill(kj > qi, _NEG_INF)
    return s


def _softmax_rows(s: torch.Tensor):
    """Safe softmax along the last axis; also returns the row max m and sum l."""
    m = s.amax(dim=-1, keepdim=True)
    e = torch.exp(s - m)
    l = e.sum(dim=-1, keepdim=True)
    return e / l, m.squeeze(-1), l.squeeze(-1)


def _row_groups(nq: int, row_chunk: int | None):
    step = nq if not row_chunk else max(1, int(row_chunk))
    for r0 in range(0, nq, step):
        yield r0, min(nq, r0 + step)


def attention_probs(q, k, scale: float, causal: bool) -> torch.Tensor:
    """P = softmax(scale * Q K^T) row by row, as a dense [B, H, Nq, Nk] tensor.

    Only for small inputs (the whole N x N matrix is materialised).
    """
    q, k = _f64(q), _f64(k)
    _check_dense(q, k, k, causal)
    out = []
    for b in range(q.shape[0]):
        s = _scores(q[b].transpose(0, 1), k[b].transpose(0, 1), scale, 0, causal)
        out.append(_softmax_rows(s)[0])
    return torch.stack(out)


def attention_forward(q, k, v, scale: float, causal: bool, row_chunk: int | None = 1024):
    """O = softmax(scale * Q K^T) V and LSE = m + ln(l) per query row.

    q: [B, Nq, H, d]; k, v: [B, Nk, H, d].  Returns (O [B, Nq, H, d],
    LSE [B, H, Nq]) in float64.  Natural-log units of the scaled scores.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check_dense(q, k, v, causal)
    B, Nq, H, d = q.shape
    o = torch.empty(B, Nq, H, d, dtype=torch.float64)
    lse = torch.empty(B, H, Nq, dtype=torch.float64)
    for b in range(B):
        qb = q[b].transpose(0, 1)  # [H, Nq, d]
        kb = k[b].transpose(0, 1)
        vb = v[b].transpose(0, 1)
        for r0, r1 in _row_groups(Nq, row_chunk):
            kend = r1 if causal else kb.shape[1]  # keys past r1-1 are masked for every row here
            s = _scores(qb[:, r0:r1], kb[:, :kend], scale, r0, causal)
            p, m, l = _softmax_rows(s)
            o[b, r0:r1] = torch.matmul(p, vb[:, :kend]).transpose(0, 1)
            lse[b, :, r0:r1] = m + torch.log(l)
    return o, lse


def attention_backward(q, k, v, dout, scale: float, causal: bool,
                       row_chunk: int | None = 1024):
    """Gradients of L = sum(O * dO) with respect to Q, K and V.

    P is recomputed from the definition for each group of query rows, then:
    dV = P^T dO, dP = dO V^T, D = rowsum(P * dP), dS = P * (dP - D),
    dQ = scale * dS K, dK = scale * dS^T Q.  Returns (dq, dk, dv, D) in
    float64, dq/dk/dv as [B, N, H, d] and D as [B, H, Nq].
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    _check_dense(q, k, v, causal)
    if do.shape != q.shape:
        raise ValueError("dout must have q's shape")
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    dq = torch.zeros(B, Nq, H, d, dtype=torch.float64)
    dk = torch.zeros(B, Nk, H, d, dtype=torch.float64)
    dv = torch.zeros(B, Nk, H, d, dtype=torch.float64)
    dvec = torch.empty(B, H, Nq, dtype=torch.float64)
    for b in range(B):
        qb, kb, vb, dob = (t[b].transpose(0, 1) for t in (q, k, v, do))
        dkb = torch.zeros(H, Nk, d, dtype=torch.float64)
        dvb = torch.zeros(H, Nk, d, dtype=torch.float64)
        for r0, r1 in _row_groups(Nq, row_chunk):
            kend = r1 if causal else Nk
            s = _scores(qb[:, r0:r1], kb[:, :kend], scale, r0, causal)
            p = _softmax_rows(s)[0]                                  # [H, R, K]
            do_r = dob[:, r0:r1]
            dvb[:, :kend] += torch.matmul(p.transpose(-1, -2), do_r)
            dp = torch.matmul(do_r, vb[:, :kend].transpose(-1, -2))  # [H, R, K]
            drow = (p * dp).sum(dim=-1, keepdim=True)
            ds = p * (dp - drow)
            dq[b, r0:r1] = (scale * torch.matmul(ds, kb[:, :kend])).transpose(0, 1)
            dkb[:, :kend] += scale * torch.matmul(ds.transpose(-1, -2), qb[:, r0:r1])
            dvec[b, :, r0:r1] = drow.squeeze(-1)
        dk[b] = dkb.transpose(0, 1)
        dv[b] = dvb.transpose(0, 1)
    return dq, dk, dv, dvec


def online_softmax_forward(q, k, v, scale: float, causal: bool,
                           boundaries: Sequence[int]):
    """Forward pass by the online-softmax update over key blocks.

    ``boundaries`` = [0, b1, ..., Nk] splits the keys into blocks.  For each
    block with scores S', row max m', P~' = exp(S' - m') and row sum l':
        m_new = max(m, m');  l <- e^(m - m_new) l + e^(m' - m_new) l'
        O <- e^(m - m_new) O + e^(m' - m_new) P~' V'
    starting from m = -inf, l = 0, O = 0; O is divided by l once at the end.
    A block whose keys are all masked for a row contributes nothing to it.
    Returns (O [B, Nq, H, d], LSE [B, H, Nq]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check_dense(q, k, v, causal)
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    bnd = [int(x) for x in boundaries]
    if bnd[0] != 0 or bnd[-1] != Nk or any(b1 <= b0 for b0, b1 in zip(bnd, bnd[1:])):
        raise ValueError("boundaries must rise strictly from 0 to Nk")
    o_out = torch.empty(B, Nq, H, d, dtype=torch.float64)
    lse_out = torch.empty(B, H, Nq, dtype=torch.float64)
    for b in range(B):
        qb, kb, vb = (t[b].transpose(0, 1) for t in (q, k, v))
        m = torch.full((H, Nq), _NEG_INF, dtype=torch.float64)
        l = torch.zeros(H, Nq, dtype=torch.float64)
        acc = torch.zeros(H, Nq, d, dtype=torch.float64)
        for j0, j1 in zip(bnd, bnd[1:]):
            s = scale * torch.matmul(qb, kb[:, j0:j1].transpose(-1, -2))
            if causal:
                qi = torch.arange(Nq).unsqueeze(1)
                kj = torch.arange(j0, j1).unsqueeze(0)
                s = s.masked_fill(kj > qi, _NEG_INF)
            m_blk = s.amax(dim=-1)
            live = m_blk > _NEG_INF            # rows with at least one visible key here
            m_safe = torch.where(live, m_blk, torch.zeros_like(m_blk))
            p_t = torch.exp(s - m_safe.unsqueeze(-1))     # masked entries -> 0
            l_blk = p_t.sum(dim=-1)
            m_new = torch.maximum(m, m_blk)
            seen = m_new > _NEG_INF
            base = torch.where(seen, m_new, torch.zeros_like(m_new))
            f_old = torch.where(m > _NEG_INF, torch.exp(m - base), torch.zeros_like(m))
            f_blk = torch.where(live, torch.exp(m_blk - base), torch.zeros_like(m_blk))
            l = f_old * l + f_blk * l_blk
            acc = f_old.unsqueeze(-1) * acc + f_blk.unsqueeze(-1) * torch.matmul(p_t, vb[:, j0:j1])
            m = m_new
        o_out[b] = (acc / l.unsqueeze(-1)).transpose(0, 1)
        lse_out[b] = m + torch.log(l)
    return o_out, lse_out


def _cu_list(cu) -> list[int]:
    vals = [int(x) for x in (cu.tolist() if isinstance(cu, torch.Tensor) else cu)]
    if not vals or vals[0] != 0 or any(b < a for a, b in zip(vals, vals[1:])):
        raise ValueError("cu_seqlens must start at 0 and never decrease")
    return vals


def attention_forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                             scale: float, causal: bool, row_chunk: int | None = 1024):
    """Packed variable-length forward: each sequence attends only to itself.

    q: [total_q, H, d]; k, v: [total_k, H, d]; sequence s owns rows
    cu_q[s]:cu_q[s+1] of q and cu_k[s]:cu_k[s+1] of k and v.  Returns
    (O [total_q, H, d], LSE [nseq, H, max_seqlen_q]); LSE rows at or past a
    sequence's length are NaN (they do not exist).
    """
    cq, ck = _cu_list(cu_seqlens_q), _cu_list(cu_seqlens_k)
    if len(cq) != len(ck):
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same length")
    q, k, v = _f64(q), _f64(k), _f64(v)
    nseq = len(cq) - 1
    H, d = q.shape[1], q.shape[2]
    o = torch.zeros(q.shape, dtype=torch.float64)
    lse = torch.full((nseq, H, max_seqlen_q), float("nan"), dtype=torch.float64)
    for s in range(nseq):
        q0, q1, k0, k1 = cq[s], cq[s + 1], ck[s], ck[s + 1]
        if q1 == q0:
            continue
        if q1 - q0 > max_seqlen_q:
            raise ValueError("a sequence is longer than max_seqlen_q")
        os_, ls_ = attention_forward(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1],
                                     scale, causal, row_chunk)
        o[q0:q1] = os_[0]
        lse[s, :, : q1 - q0] = ls_[0]
    return o, lse


def attention_backward_varlen(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, scale: float,
                              causal: bool, row_chunk: int | None = 1024):
    """Packed variable-length backward; returns (dq, dk, dv) shaped like q, k, v."""
    cq, ck = _cu_list(cu_seqlens_q), _cu_list(cu_seqlens_k)
    if len(cq) != len(ck):
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same length")
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    dq = torch.zeros(q.shape, dtype=torch.float64)
    dk = torch.zeros(k.shape, dtype=torch.float64)
    dv = torch.zeros(v.shape, dtype=torch.float64)
    for s in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[s], cq[s + 1], ck[s], ck[s + 1]
        if q1 == q0 or k1 == k0:
            continue
        g = attention_backward(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1],
                               do[None, q0:q1], scale, causal, row_chunk)
        dq[q0:q1], dk[k0:k1], dv[k0:k1] = g[0][0], g[1][0], g[2][0]
    return dq, dk, dv

