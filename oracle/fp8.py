"""FP8 (e4m3) attention forward with a random Hadamard rotation of Q and K, float64 on the CPU.

TEST INFRASTRUCTURE (see the package docstring): only the tests, the smoke
check and the CPU-baseline leg of the benchmark use this module.

Sources (page title, then the section on that page):

* The low-precision forward and its outlier remedy: Q and K are multiplied by a
  random orthogonal matrix J (J J^T = I), which leaves S = Q K^T = (QJ)(KJ)^T
  unchanged while spreading outliers concentrated in a few dimensions over all
  of them, so that FP8 quantisation loses less: "LLM Systems 22: Flash
  Attention", §4.1.3 Low-precision - FP8.  The page names the Hadamard
  transform as J.
* Everything after quantisation is the definition of attention with the safe
  softmax and LSE = m + ln(l): "08 · FlashAttention", §一 and §二; "LLM Systems
  22: Flash Attention", §3.2.

Readings taken where the pages are silent (each one is a choice, stated):

* Format: the pages say "FP8"; read as the OCP 8-bit E4M3 format (1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits, subnormals, largest finite
  value 448, no infinities, S.1111.111 is NaN).  Encoding rounds to nearest,
  ties to the even code, and saturates at +-448.
* J = diag(sigma) H_d / sqrt(d): H_d is the Sylvester Hadamard matrix
  (H[i, j] = (-1)^popcount(i & j)) and sigma in {+1, -1}^d are random signs,
  an input.  The rotated tensors are kept unnormalised, Qh = Q diag(sigma) H_d
  (likewise Kh), and the 1/d that restores J's normalisation goes into the
  score scale: Qh Kh^T = d Q K^T.  V is not rotated.
* Scales: one per block of 64 consecutive rows of each (batch, head) and
  tensor, a power of two, s = 2^ceil(log2(amax / 448)) over the block's
  rotated values (s = 1 when amax = 0); codes = e4m3(x / s).  Dividing by a
  power of two is exact, so the code depends only on the value x.
* Scores S_ij = scale * s_q(i) * s_k(j) / d * (q8_i . k8_j), decoded codes;
  V row j is s_v(j) * v8_j.
* P~ = exp(S - m) with m a per-row reference maximum; the P V product uses
  p8 = e4m3(2^(8 - tau) * P~) and O = sum_j p8_j s_v(j) v8_j / (2^(8 - tau) l),
  where l = sum_j P~_j is the unquantised row sum; LSE = m + ln(l).  The keys
  are visited in blocks of 64 ("08 · FlashAttention", §二), so P~ is rounded
  relative to the reference at that block and earlier blocks are rescaled
  after rounding: the one-pass kernel cannot know the final maximum when it
  rounds.
* The reference moves conditionally, the online-softmax variant of "LLM
  Systems 22: Flash Attention", §4.2.1, which skips most rescaling (the page
  gives no rule; read as a threshold): a block whose row maximum exceeds the
  reference by more than tau * ln 2 (tau = 4: a factor 16) makes that maximum
  the new reference and rescales the row's sums; otherwise the reference
  stays, P~ <= 2^tau, and 2^(8 - tau) P~ <= 256 stays inside e4m3's range.
  tau = 0 is the classic update (a new maximum always becomes the reference).
  A decision within the tie window of the threshold may go either way in a
  kernel's fp32 arithmetic and changes how later probabilities round, so such
  a row's O is not unique: its slack is infinite (LSE does not depend on the
  reference and keeps its bound).

Layout: q, k, v [B, N, H, d]; codes the same, uint8; scales [B, H, nblk]; O
[B, Nq, H, d]; LSE [B, H, Nq].
"""

from __future__ import annotations

import math

import torch

_NEG_INF = float("-inf")
E4M3_MAX = 448.0
RESCALE_LOG2 = 4.0       # tau: the reference maximum moves when exceeded by more than 2^tau
KEY_BLOCK = 64           # keys per block of the online pass (the kernel's key tile)
QUANT_ROWS = 64          # rows per quantisation scale


def _f64(x: torch.Tensor) -> torch.Tensor:
    return x.detach().to(device="cpu", dtype=torch.float64)


# --------------------------------------------------------------------- e4m3 codec

def e4m3_decode(codes: torch.Tensor) -> torch.Tensor:
    """Value of each code: (-1)^s 2^(e-7) (1 + m/8), subnormal (e = 0) 2^-6 m/8."""
    c = codes.to(torch.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = (c & 7).to(torch.float64)
    normal = torch.ldexp(1.0 + m / 8.0, (e - 7).to(torch.float64))
    sub = torch.ldexp(m / 8.0, torch.full_like(m, -6.0))
    v = torch.where(e == 0, sub, normal)
    v = torch.where((e == 15) & ((c & 7) == 7), torch.full_like(v, float("nan")), v)
    return torch.where(s == 1, -v, v)


def _binade(a: torch.Tensor) -> torch.Tensor:
    """floor(log2(a)) for a > 0, exactly (from the binary exponent); -6 for a = 0."""
    _, ex = torch.frexp(torch.where(a > 0, a, torch.ones_like(a)))
    return torch.where(a > 0, (ex - 1).to(torch.float64), torch.full_like(a, -6.0))


def e4m3_encode(x: torch.Tensor) -> torch.Tensor:
    """Nearest e4m3 code, ties to the even code, saturating at +-448 (float64 in)."""
    x = _f64(x)
    if torch.isnan(x).any():
        raise ValueError("NaN has no reading here")
    a = x.abs().clamp(max=E4M3_MAX)
    # spacing of the representable values around a: 2^(e-3) for a in [2^e, 2^(e+1)),
    # e >= -6; below 2^-6 (subnormals) the spacing stays 2^-9
    e = _binade(a).clamp(min=-6.0)
    quantum = torch.ldexp(torch.ones_like(a), (e - 3))
    # torch.round is round-half-to-even on the integer multiple of the quantum
    q = torch.round(a / quantum) * quantum          # at most 448: a <= 448 and 448 is a code
    # code of the non-negative value q
    qe = _binade(q)
    is_sub = q < 2.0 ** -6
    mant_sub = torch.round(q / 2.0 ** -9)
    mant_norm = torch.round((q / torch.ldexp(torch.ones_like(q), qe) - 1.0) * 8.0)
    code = torch.where(is_sub, mant_sub, (qe + 7) * 8 + mant_norm).to(torch.int64)
    code = torch.where(torch.signbit(x), code | 128, code)
    # a negative value that rounds to zero keeps its sign bit (-0, code 0x80)
    return code.to(torch.uint8)


def e4m3_step(codes: torch.Tensor) -> torch.Tensor:
    """Distance from |decode(code)| to the next larger representable magnitude."""
    c = codes.to(torch.int64) & 127
    nxt = (c + 1).clamp(max=126)
    return e4m3_decode(nxt) - e4m3_decode(c)


def e4m3_near_tie(x: torch.Tensor, rel: float = 1e-5, atol=0.0) -> torch.Tensor:
    """True where |x| lies within max(rel |x|, atol) of a midpoint between two codes.

    There a difference in how x was computed (its rounding error, at most that
    distance) may flip the code to its neighbour; both neighbours are then
    correct encodings of x.  atol may be a tensor broadcastable to x.
    """
    a = _f64(x).abs().clamp(max=E4M3_MAX)
    lo = e4m3_decode(e4m3_encode(a))
    step_up = e4m3_step(e4m3_encode(a))
    below = e4m3_decode((e4m3_encode(a).to(torch.int64) - 1).clamp(min=0).to(torch.uint8))
    mid_up = lo + 0.5 * step_up
    mid_dn = 0.5 * (lo + below)
    tol = torch.maximum(rel * a.clamp(min=2.0 ** -9), torch.as_tensor(atol, dtype=torch.float64))
    return ((a - mid_up).abs() <= tol) | (((a - mid_dn).abs() <= tol) & (lo > 0))


# ---------------------------------------------------------------- the rotation

def hadamard(d: int) -> torch.Tensor:
    """Sylvester Hadamard matrix of order d (a power of two), float64, entries +-1."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = torch.ones(1, 1, dtype=torch.float64)
    while h.shape[0] < d:
        h = torch.cat([torch.cat([h, h], 1), torch.cat([h, -h], 1)], 0)
    return h


def rotate(x: torch.Tensor, signs: torch.Tensor) -> torch.Tensor:
    """x diag(sigma) H_d along the last axis (unnormalised: J = this / sqrt(d))."""
    x = _f64(x)
    d = x.shape[-1]
    return torch.matmul(x * _f64(signs).reshape(d), hadamard(d))


def quantize_e4m3(x: torch.Tensor, signs: torch.Tensor | None = None,
                  block_rows: int | None = QUANT_ROWS):
    """Power-of-two scales and e4m3 codes of x (rotated if signs are given).

    One scale per block of ``block_rows`` consecutive rows of each (batch, head)
    (None: one block of all rows), s = 2^ceil(log2(amax / 448)) over the block's
    values (1 for an all-zero block).  Returns (codes uint8 [B, N, H, d], scales
    float64 [B, H, nblk], scaled float64 [B, N, H, d] = x / s, the values that
    were rounded).
    """
    xr = rotate(x, signs) if signs is not None else _f64(x)
    B, N, H, d = xr.shape
    rows = N if block_rows is None else int(block_rows)
    nblk = max(1, -(-N // rows))
    pad = nblk * rows - N
    xp = torch.cat([xr, torch.zeros(B, pad, H, d, dtype=torch.float64)], 1) if pad else xr
    amax = xp.abs().reshape(B, nblk, rows, H, d).amax(dim=(2, 4)).transpose(1, 2)   # [B, H, nblk]
    e = torch.ceil(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)) / E4M3_MAX))
    s = torch.where(amax > 0, torch.ldexp(torch.ones_like(amax), e), torch.ones_like(amax))
    scaled = xr / row_scales(s, N, rows).transpose(1, 2)[..., None]
    return e4m3_encode(scaled), s, scaled


def row_scales(s: torch.Tensor, n: int, rows: int) -> torch.Tensor:
    """Per-block scales [B, H, nblk] -> the scale of every row, [B, H, n].
    Scales given as [B, H] are one block of all rows."""
    s = _f64(s)
    if s.dim() == 2:
        return s[:, :, None].expand(s.shape[0], s.shape[1], n)
    return s.repeat_interleave(int(rows), dim=2)[:, :, :n]


# ------------------------------------------------------------- fp8 attention

def fp8_attention_forward(q8, k8, v8, sq, sk, sv, qk_scale: float, causal: bool,
                          tie_rel: float = 1e-5, q_scaled=None, k_scaled=None, v_scaled=None,
                          q_tie_atol=0.0, k_tie_atol=0.0, block: int | None = KEY_BLOCK,
                          scale_rows: int = QUANT_ROWS, rescale_log2: float = RESCALE_LOG2,
                          p_tie_rel: float | None = None):
    """Attention over decoded e4m3 codes with the P V product on e4m3 probabilities.

    q8 [B, Nq, H, d], k8/v8 [B, Nk, H, d] uint8 codes; sq, sk, sv [B, H, nblk]
    scales, one per block of ``scale_rows`` rows; S_ij = qk_scale * sq_i * sk_j *
    (q8_i . k8_j) and V row j is sv_j * v8_j.  The keys are visited in blocks of
    ``block`` (None: one block) with the online softmax ("08 · FlashAttention",
    §二) and a per-row reference maximum m: a block whose row maximum m_blk
    exceeds m by more than rescale_log2 * ln 2 makes it the reference, and the
    row's earlier sums are rescaled by e^(m - m_blk) ("LLM Systems 22: Flash
    Attention", §4.2.1: most rescaling is skipped).  Per block P~ = exp(S - m)
    <= 2^rescale_log2 is rounded as e4m3(2^(8 - rescale_log2) P~) for the P V
    product, and the row sum l keeps the unrounded P~.  Rounding P~ at the
    current reference rather than the final maximum is what a one-pass kernel
    can do; with one block and rescale_log2 = 0 the two agree.

    Returns (O, LSE, slack_o, slack_lse): slack bounds, to first order, how far
    O and LSE may move when codes that sit at a near-tie (P~, and Q, K, V when
    their pre-rounding values q_scaled/k_scaled/v_scaled are given) round to the
    neighbouring code; a code counts as near a tie within max(tie_rel |x|,
    *_tie_atol) of a midpoint (P codes: p_tie_rel |x|, default tie_rel).  A row with a reference decision within
    tie_rel (|m| + |m_blk|) of the threshold gets slack_o = inf (either
    decision is a correct execution, and they round later probabilities
    differently).
    """
    qd, kd, vd = e4m3_decode(q8), e4m3_decode(k8), e4m3_decode(v8)
    B, Nq, H, d = qd.shape
    Nk = kd.shape[1]
    if causal and Nq != Nk:
        raise ValueError("causal attention needs Nq == Nk")
    sq, sk, sv = _f64(sq), _f64(sk), _f64(sv)
    o = torch.zeros(B, Nq, H, d, dtype=torch.float64)
    lse = torch.full((B, H, Nq), _NEG_INF, dtype=torch.float64)
    slack_o = torch.zeros_like(o)
    slack_l = torch.zeros_like(lse)
    if Nk == 0:
        return o, lse, slack_o, slack_l
    bs = Nk if block is None else int(block)
    p_scale = 2.0 ** (8.0 - rescale_log2)   # e4m3(p_scale * P~) <= 256
    thr = rescale_log2 * math.log(2.0)
    p_tie = tie_rel if p_tie_rel is None else p_tie_rel

    def tie_steps(scaled, codes, atol=0.0):
        if scaled is None:
            return torch.zeros(codes.shape, dtype=torch.float64)
        return e4m3_near_tie(scaled, tie_rel, atol).to(torch.float64) * e4m3_step(codes)

    tq, tk = tie_steps(q_scaled, q8, q_tie_atol), tie_steps(k_scaled, k8, k_tie_atol)
    tv = tie_steps(v_scaled, v8)
    rq = row_scales(sq, Nq, scale_rows)                                # [B, H, Nq]
    rk = row_scales(sk, Nk, scale_rows)
    rv = row_scales(sv, Nk, scale_rows)
    for b in range(B):
        for h in range(H):
            c = qk_scale * torch.outer(rq[b, h], rk[b, h])            # [Nq, Nk]
            qh, kh = qd[b, :, h], kd[b, :, h]
            vh = vd[b, :, h] * rv[b, h][:, None]                        # V in its own units
            tvh = tv[b, :, h] * rv[b, h][:, None]
            s = c * torch.matmul(qh, kh.transpose(0, 1))              # [Nq, Nk]
            # |dS| from Q/K codes at a near-tie flipping by one step
            ds = c * (torch.matmul(tq[b, :, h], kh.abs().transpose(0, 1))
                      + torch.matmul(qh.abs(), tk[b, :, h].transpose(0, 1)))
            if causal:
                vis = torch.arange(Nk).unsqueeze(0) <= torch.arange(Nq).unsqueeze(1)
                s = s.masked_fill(~vis, _NEG_INF)
                ds = ds.masked_fill(~vis, 0.0)
            m_fin = s.amax(dim=-1, keepdim=True)
            live = m_fin > _NEG_INF
            m_fin0 = torch.where(live, m_fin, torch.zeros_like(m_fin))
            # the online pass over key blocks
            m = torch.full((Nq, 1), _NEG_INF, dtype=torch.float64)
            acc = torch.zeros(Nq, d, dtype=torch.float64)
            l = torch.zeros(Nq, 1, dtype=torch.float64)
            # P-tie steps * |v| and p8 * V-tie steps, rescaled like acc (units of the
            # current reference, which may stay below the row's true maximum)
            tie_p = torch.zeros(Nq, d, dtype=torch.float64)
            tie_v = torch.zeros(Nq, d, dtype=torch.float64)
            amb = torch.zeros(Nq, 1, dtype=torch.bool)        # a reference decision at a near-tie
            for j0 in range(0, Nk, bs):
                sb = s[:, j0:j0 + bs]
                m_blk = sb.amax(dim=-1, keepdim=True)
                fin = (m > _NEG_INF) & (m_blk > _NEG_INF)
                rise = torch.where(fin, m_blk - m, torch.zeros_like(m))
                if thr > 0:   # with thr = 0 both choices give the same reference
                    amb |= fin & ((rise - thr).abs() <= tie_rel * (m.abs() + m_blk.abs()))
                m_new = torch.where(m_blk > m + thr, m_blk, m)          # the reference moves
                m_ref = torch.where(m_new > _NEG_INF, m_new, torch.zeros_like(m_new))
                alpha = torch.exp(m - m_ref)
                pt = torch.exp(sb - m_ref)                            # P~ <= 2^tau
                p8 = e4m3_encode(p_scale * pt)
                pq = e4m3_decode(p8)
                acc = alpha * acc + torch.matmul(pq, vh[j0:j0 + bs])
                l = alpha * l + pt.sum(dim=-1, keepdim=True)
                m = m_new
                tp = e4m3_near_tie(p_scale * pt, p_tie).to(torch.float64) * e4m3_step(p8)
                tie_p = alpha * tie_p + torch.matmul(tp, vh[j0:j0 + bs].abs())
                tie_v = alpha * tie_v + torch.matmul(pq, tvh[j0:j0 + bs])
            linv = torch.where(live, 1.0 / l, torch.zeros_like(l))
            o[b, :, h] = acc / p_scale * linv
            lse[b, h] = torch.where(live, m + torch.log(l), torch.full_like(m, _NEG_INF)).squeeze(-1)
            # slack: P codes at a near-tie, V codes at a near-tie, and dS (first order)
            p_true = torch.exp(s - m_fin0) * torch.where(live, 1.0 / torch.exp(s - m_fin0).sum(-1, keepdim=True), torch.zeros_like(l))
            vabs = vh.abs()
            so = (tie_p + tie_v) / p_scale * linv
            dev = torch.matmul(p_true * ds, vabs) + (p_true * ds).sum(-1, keepdim=True) * o[b, :, h].abs()
            slack_o[b, :, h] = torch.where(amb, torch.full_like(so, math.inf), so + dev)
            slack_l[b, h] = (p_true * ds).sum(dim=-1)
    return o, lse, slack_o, slack_l


def fp32_rotation_error(x: torch.Tensor, signs: torch.Tensor, s: torch.Tensor,
                        block_rows: int = QUANT_ROWS) -> torch.Tensor:
    """Bound on |fp32 rotation - exact| / s per row: a fast Walsh-Hadamard
    transform in fp32 rounds once per butterfly stage, each rounding at most
    2^-24 of a partial sum bounded by the row's L1 norm, log2(d) stages.
    s: the scales [B, H, nblk] of blocks of block_rows rows.  Returns [B, N, H, 1]."""
    x = _f64(x)
    B, N, H, d = x.shape
    l1 = (x * _f64(signs).reshape(d)).abs().sum(dim=-1, keepdim=True)
    return math.log2(d) * 2.0 ** -24 * l1 / row_scales(s, N, block_rows).transpose(1, 2)[..., None]


def fp8_forward(q, k, v, signs, scale: float, causal: bool, rotate_qk: bool = True,
                tie_rel: float = 1e-5, fp32_rotation: bool = False):
    """The whole FP8 forward from bf16/float inputs: rotate, quantise, attend.

    With fp32_rotation, codes of Q and K within twice the fp32 rotation's
    rounding bound of a midpoint count as near a tie (a kernel that rotates in
    fp32 may round them either way).
    Returns (O, LSE, slack_o, slack_lse, (q8, k8, v8), (sq, sk, sv)).
    """
    d = q.shape[-1]
    sg = signs if rotate_qk else None
    q8, sq, qs = quantize_e4m3(q, sg)
    k8, sk, ks = quantize_e4m3(k, sg)
    v8, sv, vs = quantize_e4m3(v, None)
    qk_scale = scale / d if rotate_qk else scale
    qa = ka = 0.0
    if fp32_rotation and rotate_qk:
        qa = 2.0 * fp32_rotation_error(q, signs, sq)
        ka = 2.0 * fp32_rotation_error(k, signs, sk)
    o, lse, so, sl = fp8_attention_forward(q8, k8, v8, sq, sk, sv, qk_scale, causal, tie_rel,
                                           qs, ks, vs, qa, ka)
    return o, lse, so, sl, (q8, k8, v8), (sq, sk, sv)


def rmse(a: torch.Tensor, b: torch.Tensor) -> float:
    """Root-mean-square difference."""
    return math.sqrt(float(((_f64(a) - _f64(b)) ** 2).mean()))
