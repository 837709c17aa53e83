"""An a-priori error model of the FP8 forward against exact attention.

It uses neither the FP8 oracle's blocked algorithm nor any of its design
choices (block sizes, the rescale threshold, how P is normalised): only the
exact float64 attention, the rotation ("LLM Systems 22: Flash Attention",
§4.1.3; pinned to scipy's Hadamard matrix) and the spacing of the e4m3 format.

Model.  Every e4m3 rounding -- of the rotated Q and K, of V, of the
probabilities P -- moves a value by at most half the code spacing h at that
value, and is taken as an independent error uniform on [-h, h] (variance h^2/3).
For a power-of-two scale s the spacing of e4m3 at |x| (in x's units) is
2^(floor(log2|x|) - 3) whatever s is, so h(x) = 2^(floor(log2|x|) - 4); only
below the normal range (|x/s| < 2^-6) does s matter, where h = s 2^-10, bounded
here with the largest scale any block of the head can get (amax over the head).
P is rounded relative to some reference; its relative half-step is at most
2^-4 (normal codes), with an absolute floor of 2^-14 for subnormal codes.

Propagating those errors to first order through O = softmax(S) V:
  scores  dS_ij = c (dq_i . k_j + q_i . dk_j),  c the score scale (scale/d
          after the unnormalised rotation), which moves O_i by
          sum_j P_ij dS_ij (v_j - O_i): the q part is dq_i . W_i with
          W_i[a, c'] = sum_j P_ij k_ja (v_jc' - O_ic'), the k part is a sum of
          independent terms over j;
  values  sum_j P_ij dv_jc;
  probs   sum_j dP_ij (v_jc or v_jc - O_ic, depending on how O is normalised:
          both are covered by v_jc^2 + O_ic^2).
The variance of each element is the sum of those terms; sigma is its root.
A correct FP8 forward then has |O - O_exact| <= 6 sigma + (bf16 output
rounding 2^-8 |O|) + 1e-5 for all but a ~1e-9 fraction of elements (the
errors are sums of many small independent terms); a shared mistake (a
wrong scale, a missing normalisation, V rotated too) moves O by far more.

LSE depends only on the scores: sigma_lse^2 = c^2 (sum_a Var dq_a (sum_j P_j k_ja)^2
+ sum_j P_j^2 sum_a q_a^2 Var dk_ja).
"""

from __future__ import annotations

import math

import torch

import oracle as dense
from oracle.fp8 import rotate

E4M3_MAX = 448.0


def half_step(x: torch.Tensor, s_max: torch.Tensor) -> torch.Tensor:
    """Half the e4m3 spacing at |x| for a power-of-two scale <= s_max (broadcast)."""
    a = x.abs()
    e = torch.floor(torch.log2(a.clamp(min=1e-300)))
    h = torch.ldexp(torch.ones_like(a), e - 4)
    return torch.maximum(torch.where(a > 0, h, torch.zeros_like(h)), s_max * 2.0 ** -10)


def _head_scale(x: torch.Tensor) -> torch.Tensor:
    """Largest power-of-two scale any block of each (batch, head) can get: [B, 1, H, 1]."""
    amax = x.abs().amax(dim=(1, 3), keepdim=True)
    e = torch.ceil(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)) / E4M3_MAX))
    return torch.ldexp(torch.ones_like(amax), e)


def fp8_sigma(q, k, v, signs, scale: float, causal: bool, rotate_qk: bool = True, row_chunk: int = 256):
    """Exact O, LSE, the model's standard deviations sigma_o [B, Nq, H, d] and
    sigma_lse [B, H, Nq], and the largest standard deviation of one visible score
    of each row, sigma_s [B, H, Nq] (float64, CPU).  The first-order model holds
    where sigma_s is small (below ~0.25 the second-order remainder is a few per
    cent); unrotated inputs with outlier channels leave that regime."""
    q, k, v = (t.detach().to("cpu", torch.float64) for t in (q, k, v))
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    qr = rotate(q, signs) if rotate_qk else q
    kr = rotate(k, signs) if rotate_qk else k
    c = scale / d if rotate_qk else scale
    vq = half_step(qr, _head_scale(qr)) ** 2 / 3
    vk = half_step(kr, _head_scale(kr)) ** 2 / 3
    vv = half_step(v, _head_scale(v)) ** 2 / 3
    o_ex, lse_ex = dense.attention_forward(q, k, v, scale, causal)
    sig_o = torch.zeros(B, Nq, H, d, dtype=torch.float64)
    sig_l = torch.zeros(B, H, Nq, dtype=torch.float64)
    sig_s = torch.zeros(B, H, Nq, dtype=torch.float64)
    p_rel = 2.0 ** -8 / 3        # (2^-4)^2 / 3
    p_abs = 2.0 ** -28 / 3       # (2^-14)^2 / 3
    for b in range(B):
        for h in range(H):
            kh, vh, qh = kr[b, :, h], v[b, :, h], qr[b, :, h]
            for i0 in range(0, Nq, row_chunk):
                i1 = min(Nq, i0 + row_chunk)
                s = c * qh[i0:i1] @ kh.T
                if causal:
                    vis = torch.arange(Nk)[None, :] <= torch.arange(i0, i1)[:, None]
                    s = s.masked_fill(~vis, -math.inf)
                p = torch.softmax(s, dim=-1)                                   # [R, Nk]
                o = p @ vh                                                     # [R, d]
                p2 = p * p
                # q part: W_i[a, c'] = sum_j P_ij k_ja (v_jc' - O_ic')
                pk = p @ kh                                                    # [R, d]
                w = torch.einsum("rj,ja,jc->rac", p, kh, vh) - pk[:, :, None] * o[:, None, :]
                t_q = c * c * torch.einsum("ra,rac->rc", vq[b, i0:i1, h], w * w)
                # k part: sum_j P_ij^2 (sum_a q_ia^2 Var dk_ja) (v_jc - O_ic)^2
                g = p2 * ((qh[i0:i1] ** 2) @ vk[b, :, h].T)                      # [R, Nk]
                t_k = c * c * (g @ vh ** 2 - 2 * o * (g @ vh) + o ** 2 * g.sum(-1, keepdim=True))
                t_v = p2 @ vv[b, :, h]
                pw = p2 * p_rel + p_abs * (p > 0)
                t_p = pw @ vh ** 2 + o ** 2 * pw.sum(-1, keepdim=True)
                sig_o[b, i0:i1, h] = (t_q + t_k + t_v + t_p).sqrt()
                vs = c * c * (vq[b, i0:i1, h] @ (kh ** 2).T + (qh[i0:i1] ** 2) @ vk[b, :, h].T)
                sig_s[b, h, i0:i1] = torch.where(p > 0, vs, torch.zeros_like(vs)).amax(-1).sqrt()
                l_q = (vq[b, i0:i1, h] * pk ** 2).sum(-1)
                l_k = (p2 * ((qh[i0:i1] ** 2) @ vk[b, :, h].T)).sum(-1)
                sig_l[b, h, i0:i1] = (c * c * (l_q + l_k)).sqrt()
    return o_ex, lse_ex, sig_o, sig_l, sig_s


K_SIGMA = 6.0
SIGMA_S_MAX = 0.25


def check_apriori(o, lse, o_ex, lse_ex, sig_o, sig_l, sig_s, what=""):
    """On rows in the model's regime (sigma_s <= 0.25): |O - O_exact| <= 6 sigma
    + 2^-8 |O_exact| + 1e-5 and |LSE - LSE_exact| <= 6 sigma_lse + 1e-5.
    Returns the largest ratio of an error to its bound, for O and LSE, the RMS of
    error / sigma and the fraction of rows outside the regime."""
    o = o.detach().to("cpu", torch.float64)
    lse = lse.detach().to("cpu", torch.float64)
    rows = sig_s <= SIGMA_S_MAX                                   # [B, H, Nq]
    rows_o = rows.transpose(1, 2)[..., None].expand_as(o)        # [B, Nq, H, d]
    eo = (o - o_ex).abs()[rows_o]
    bo = (K_SIGMA * sig_o + 2.0 ** -8 * o_ex.abs() + 1e-5)[rows_o]
    fin = torch.isfinite(lse_ex) & rows
    el = (lse - lse_ex).abs()[fin]
    bl = (K_SIGMA * sig_l + 1e-5)[fin]
    r_o = (eo / bo).max().item() if eo.numel() else 0.0
    r_l = (el / bl).max().item() if el.numel() else 0.0
    assert r_o <= 1.0, f"FP8 O error {r_o:.3f} of the a-priori bound {what}"
    assert r_l <= 1.0, f"FP8 LSE error {r_l:.3f} of the a-priori bound {what}"
    z = ((eo - 2.0 ** -8 * o_ex.abs()[rows_o]).clamp(min=0) / sig_o[rows_o].clamp(min=1e-12))
    rms = z.pow(2).mean().sqrt().item() if z.numel() else 0.0
    return r_o, r_l, rms, 1.0 - rows.double().mean().item()
