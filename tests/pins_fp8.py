"""Checks that tie the FP8 oracle (oracle/fp8.py) to facts outside it.

Each ``pin_*`` takes a module with the functions of oracle/fp8.py (normally
``oracle.fp8``; the mutation tests pass copies with a planted mistake).  The
facts:

* the OCP E4M3 format: the values of named codes (the format's definition:
  bias 7, three mantissa bits, 448 the largest finite value, S.1111.111 NaN),
  and encoding = the nearest code by exhaustive search, ties to the even code;
* the Sylvester Hadamard matrix is scipy's ``hadamard`` and H H^T = d I, so
  J = diag(sigma) H / sqrt(d) is orthogonal and (QJ)(KJ)^T = Q K^T ("LLM Systems
  22: Flash Attention", §4.1.3);
* with scores whose exponentials are exact powers of two, P~ quantises without
  loss and the FP8 attention must equal the float64 dense oracle (pinned on its
  own) on the decoded inputs; in general the difference is bounded by half an
  e4m3 step of each P~;
* the whole FP8 forward stays close to exact attention, and the rotation lowers
  the error when a few channels of Q and K carry outliers (the page's claim).
"""

from __future__ import annotations

import math

import numpy as np
import scipy.linalg
import torch

import oracle as dense


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64) * scale


def _signs(d, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(0, 2, (d,), generator=g).to(torch.float64) * 2 - 1


def pin_e4m3_named_codes(f):
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0,
             0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    codes = torch.tensor(sorted(known), dtype=torch.uint8)
    vals = f.e4m3_decode(codes)
    for c, v in zip(codes.tolist(), vals.tolist()):
        assert v == known[c], (hex(c), v)
    assert torch.isnan(f.e4m3_decode(torch.tensor([0x7F, 0xFF], dtype=torch.uint8))).all()
    # magnitudes rise strictly with the code; the sign bit only negates
    pos = f.e4m3_decode(torch.arange(127, dtype=torch.uint8))
    assert bool((pos[1:] > pos[:-1]).all())
    neg = f.e4m3_decode(torch.arange(128, 255, dtype=torch.uint8))
    assert torch.equal(neg, -pos)


def _nearest_bruteforce(f, x):
    """Encode by search over every finite code; ties -> even code; |x| > 448 -> 448."""
    codes = torch.arange(127, dtype=torch.uint8)
    vals = f.e4m3_decode(codes).tolist()
    out = []
    for xv in x.tolist():
        a = min(abs(xv), 448.0)
        best = min(range(127), key=lambda c: (abs(a - vals[c]), c & 1))
        out.append(best | (128 if math.copysign(1.0, xv) < 0 else 0))
    return torch.tensor(out, dtype=torch.uint8)


def pin_e4m3_encode_is_nearest(f):
    rng = np.random.default_rng(401)
    mags = np.exp(rng.uniform(np.log(1e-4), np.log(600.0), 3000))
    x = mags * rng.choice([-1.0, 1.0], mags.size)
    vals = f.e4m3_decode(torch.arange(127, dtype=torch.uint8)).numpy()
    mids = 0.5 * (vals[1:] + vals[:-1])
    x = np.concatenate([x, mids, -mids, vals, [449.0, 464.0, 500.0, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -11]])
    xt = torch.tensor(x, dtype=torch.float64)
    assert torch.equal(f.e4m3_encode(xt), _nearest_bruteforce(f, xt))


def pin_hadamard(f):
    for d in (1, 2, 4, 8, 16, 32, 64, 128):
        h = f.hadamard(d)
        assert torch.equal(h, torch.tensor(scipy.linalg.hadamard(d), dtype=torch.float64))
        assert torch.equal(h @ h.T, d * torch.eye(d, dtype=torch.float64))


def pin_rotation_keeps_scores(f):
    d = 64
    q, k = _rand((5, d), 402), _rand((7, d), 403)
    sg = _signs(d, 404)
    qr, kr = f.rotate(q, sg), f.rotate(k, sg)
    ref = d * (q @ k.T)
    assert (qr @ kr.T - ref).abs().max().item() < 1e-11 * ref.abs().max().item()
    # the rotation really mixes: a one-hot row spreads over every dimension
    e0 = torch.zeros(1, d, dtype=torch.float64)
    e0[0, 3] = 1.0
    assert bool((f.rotate(e0, sg).abs() == 1.0).all())
    # J = diag(sigma) H / sqrt(d): unit vector i goes to sigma_i times row i of H,
    # and row i of the Sylvester matrix is (-1)^popcount(i & j) over j
    for i in (0, 3, 37, 63):
        ei = torch.zeros(1, d, dtype=torch.float64)
        ei[0, i] = 1.0
        row = torch.tensor([(-1.0) ** bin(i & j).count("1") for j in range(d)], dtype=torch.float64)
        assert torch.equal(f.rotate(ei, sg)[0], float(sg[i]) * row), i


def pin_quantize_scale_and_codes(f):
    x = _rand((2, 150, 3, 64), 405, 3.0)
    x[1, :, 2] = 0.0                                    # an all-zero head: scale 1, codes 0
    x[0, 64:128, 1] *= 1e-3                             # one quiet block gets its own, smaller scale
    sg = _signs(64, 406)
    for signs in (None, sg):
        for rows in (64, None):
            codes, s, scaled = f.quantize_e4m3(x, signs, rows)
            xr = f.rotate(x, signs) if signs is not None else x
            r = 150 if rows is None else rows
            nblk = -(-150 // r)
            assert s.shape == (2, 3, nblk)
            for b in range(2):
                for h in range(3):
                    for k in range(nblk):
                        amax = xr[b, k * r:(k + 1) * r, h].abs().max().item()
                        sv = float(s[b, h, k])
                        if amax == 0.0:
                            assert sv == 1.0
                            assert int(codes[b, k * r:(k + 1) * r, h].to(torch.int64).max()) in (0, 128)
                            continue
                        m, e = math.frexp(sv)
                        assert m == 0.5, sv                 # a power of two
                        assert 224.0 < amax / sv <= 448.0, amax / sv   # the smallest such power
            if rows == 64 and signs is None:
                assert float(s[0, 1, 1]) < float(s[0, 1, 0]) / 256
            srow = f.row_scales(s, 150, r).transpose(1, 2)[..., None]
            dec = f.e4m3_decode(codes) * srow
            # each code within half a step of its value (relative 2^-4, or 2^-10 absolute in subnormals)
            err = (dec - xr).abs() / srow
            assert bool((err <= torch.maximum(xr.abs() / srow / 16, torch.full_like(err, 2.0 ** -10)) * (1 + 1e-12)).all())
            assert torch.equal(scaled * srow, xr)


def _exact_case(causal):
    """Codes for Q, K in {-1, 0, 1} (d = 8) and random representable V, scales 1."""
    g = torch.Generator().manual_seed(407)
    B, N, H, d = 2, 19, 2, 8
    qv = torch.randint(-1, 2, (B, N, H, d), generator=g).to(torch.float64)
    kv = torch.randint(-1, 2, (B, N, H, d), generator=g).to(torch.float64)
    vc = torch.randint(0, 127, (B, N, H, d), generator=g) | (torch.randint(0, 2, (B, N, H, d), generator=g) << 7)
    return qv, kv, vc.to(torch.uint8)


def pin_fp8_attention_exact_powers_of_two(f):
    # qk_scale = ln 2 and integer dot products: every P~ is 2^-k, k the distance
    # to the row's maximum (one block: the reference is the maximum), at most 10
    # here, so 2^(8 - tau) P~ >= 2^-6 is an exact e4m3 value and nothing is lost
    for causal in (False, True):
        qv, kv, v8 = _exact_case(causal)
        sc = torch.einsum("bihd,bjhd->bhij", qv, kv)
        vis = torch.ones(19, 19, dtype=torch.bool)
        if causal:
            vis = vis.tril()
        spread = sc.masked_fill(~vis, -99).amax(-1) - sc.masked_fill(~vis, 99).amin(-1)
        assert spread.max().item() <= 10
        q8, k8 = f.e4m3_encode(qv), f.e4m3_encode(kv)
        ones = torch.ones(2, 2, dtype=torch.float64)
        for sv in (1.0, 0.25):
            o, lse, _, _ = f.fp8_attention_forward(q8, k8, v8, ones, ones, ones * sv, math.log(2.0), causal)
            vd = f.e4m3_decode(v8) * sv
            o_ref, lse_ref = dense.attention_forward(qv, kv, vd, math.log(2.0), causal)
            assert (o - o_ref).abs().max().item() < 1e-12, (causal, sv)
            assert (lse - lse_ref).abs().max().item() < 1e-12, (causal, sv)
        # the scales multiply the scores
        o2, lse2, _, _ = f.fp8_attention_forward(q8, k8, v8, ones * 2.0, ones * 0.5, ones, math.log(2.0), causal)
        assert (o2 - f.fp8_attention_forward(q8, k8, v8, ones, ones, ones, math.log(2.0), causal)[0]).abs().max().item() < 1e-12
        o4, _, _, _ = f.fp8_attention_forward(q8, k8, v8, ones * 2.0, ones, ones, math.log(2.0) / 2, causal)
        assert (o4 - o2).abs().max().item() < 1e-12


def pin_fp8_running_max_worked_example(f):
    # one query (q = e_0), three keys with k_0 = 2, 1, 3 and scores c k, c = ln 3,
    # values v_0 = 1, 3, 4; keys in blocks of 2.  Block {0, 1}: running max at key 0,
    # P~ = 1, 1/3 -> e4m3(256) = 256, e4m3(85.33) = 88.  Block {2}: max rises by
    # ln 3, earlier terms scale by 1/3, P~ = 1 -> 256.  l = 1/3 + 1/9 + 1 = 13/9.
    # O_0 = ((256 * 1 + 88 * 3) / 3 + 256 * 4) / (256 * 13 / 9); LSE = 3 ln 3 + ln(13/9).
    # (Rounded at the final maximum instead: 88, 28, 256 -> a different O_0.)
    enc = f.e4m3_encode
    d = 4
    q8 = enc(torch.tensor([[[[1.0, 0, 0, 0]]]], dtype=torch.float64))
    k8 = enc(torch.tensor([[[[2.0, 0, 0, 0]], [[1.0, 0, 0, 0]], [[3.0, 0, 0, 0]]]], dtype=torch.float64))
    v8 = enc(torch.tensor([[[[1.0, 0, 0, 0]], [[3.0, 0, 0, 0]], [[4.0, 0, 0, 0]]]], dtype=torch.float64))
    one = torch.ones(1, 1, dtype=torch.float64)
    o, lse, _, _ = f.fp8_attention_forward(q8, k8, v8, one, one, one, math.log(3.0), False, block=2,
                                           rescale_log2=0.0)
    want = ((256 * 1 + 88 * 3) / 3 + 256 * 4) / (256 * 13 / 9)
    assert abs(o[0, 0, 0, 0].item() - want) < 1e-12, (o[0, 0, 0, 0].item(), want)
    assert abs(lse[0, 0, 0].item() - (3 * math.log(3.0) + math.log(13 / 9))) < 1e-12
    # one block: rounded at the final maximum
    o1, _, _, _ = f.fp8_attention_forward(q8, k8, v8, one, one, one, math.log(3.0), False, block=None,
                                          rescale_log2=0.0)
    assert abs(o1[0, 0, 0, 0].item() - (88 * 1 + 28 * 3 + 256 * 4) / (256 * 13 / 9)) < 1e-12
    assert d == q8.shape[-1]


def _one_query_case(f, keys, values):
    """q = e_0 and keys / values with only their first component set (exact codes)."""
    enc = f.e4m3_encode
    row = lambda x: [[x, 0.0, 0.0, 0.0]]
    q8 = enc(torch.tensor([[row(1.0)]], dtype=torch.float64))
    k8 = enc(torch.tensor([[row(float(x)) for x in keys]], dtype=torch.float64))
    v8 = enc(torch.tensor([[row(float(x)) for x in values]], dtype=torch.float64))
    return q8, k8, v8


def pin_fp8_conditional_rescale_worked_example(f):
    # one query, keys k = 2, 1, 3, 0, 5 with scores k ln 3, values 1, 3, 4, 2, 5, in
    # blocks of 2; tau = 4, so the reference moves only on a rise above 4 ln 2 =
    # 2.77 and P~ is rounded as e4m3(16 P~).
    #   {0, 1}: reference 2 ln 3; P~ = 1, 1/3 -> 16, e4m3(5.33) = 5.5
    #   {2, 3}: rise ln 3 = 1.10, kept; P~ = 3, 1/9 -> 48, e4m3(1.78) = 1.75
    #   {4}:    rise 3 ln 3 = 3.30, moved; earlier sums x 1/27; P~ = 1 -> 16
    # acc = (16 + 5.5*3 + 48*4 + 1.75*2) / 27 + 16*5 = 2388/27,
    # l = (1 + 1/3 + 3 + 1/9) / 27 + 1 = 283/243, O_0 = acc / (16 l) = 21492/4528,
    # LSE = ln(9 + 3 + 27 + 1 + 243) = ln 283.
    # The classic update (tau = 0) gives 343854/72448 here; a threshold read in
    # natural-log units (4 instead of 4 ln 2) keeps the reference at block {4}
    # and gives 22212/4528.
    q8, k8, v8 = _one_query_case(f, [2, 1, 3, 0, 5], [1, 3, 4, 2, 5])
    one = torch.ones(1, 1, dtype=torch.float64)
    c = math.log(3.0)
    o, lse, so, sl = f.fp8_attention_forward(q8, k8, v8, one, one, one, c, False, block=2)
    assert f.RESCALE_LOG2 == 4.0
    assert abs(o[0, 0, 0, 0].item() - 21492 / 4528) < 1e-12, o[0, 0, 0, 0].item()
    assert abs(lse[0, 0, 0].item() - math.log(283.0)) < 1e-12
    assert bool(torch.isfinite(so).all())
    o0, lse0, _, _ = f.fp8_attention_forward(q8, k8, v8, one, one, one, c, False, block=2, rescale_log2=0.0)
    assert abs(o0[0, 0, 0, 0].item() - 343854 / 72448) < 1e-12, o0[0, 0, 0, 0].item()
    assert abs(lse0[0, 0, 0].item() - math.log(283.0)) < 1e-12


def pin_fp8_rescale_near_tie_flagged(f):
    # scores 0 then 4 ln 2 (c = ln 2, keys 0 and 4), one key per block: the rise
    # is exactly the threshold, either decision is a correct execution, so O has
    # infinite slack; LSE = ln(1 + 16) either way.  A rise of 3 ln 2 is no tie.
    one = torch.ones(1, 1, dtype=torch.float64)
    c = math.log(2.0)
    q8, k8, v8 = _one_query_case(f, [0, 4], [1, 2])
    o, lse, so, sl = f.fp8_attention_forward(q8, k8, v8, one, one, one, c, False, block=1)
    assert bool(torch.isinf(so[0, 0, 0]).all())
    assert abs(lse[0, 0, 0].item() - math.log(17.0)) < 1e-12 and math.isfinite(sl[0, 0, 0].item())
    # the two executions: keep (P~ = 16 -> code 256) or move (P~ = 1 -> 16, earlier
    # sums / 16); both give O = (1 + 16 * 2) / 17 here, since every code is exact
    assert abs(o[0, 0, 0, 0].item() - 33 / 17) < 1e-12
    q8, k8, v8 = _one_query_case(f, [0, 3], [1, 2])
    o, lse, so, _ = f.fp8_attention_forward(q8, k8, v8, one, one, one, c, False, block=1)
    assert bool(torch.isfinite(so).all())
    assert abs(o[0, 0, 0, 0].item() - 17 / 9) < 1e-12 and abs(lse[0, 0, 0].item() - math.log(9.0)) < 1e-12


def pin_fp8_attention_p_rounding_bound(f):
    # random codes: the only difference from exact attention on the decoded inputs
    # is rounding c P~ to e4m3, c = 2^(8 - tau): |dP~| <= max(P~ / 16, 2^-10 / c)
    # (half a step: relative 2^-4 for normal codes, 2^-10 below 2^-6); every P~
    # is scaled by e^(m_ref - m_final) <= 1 and the row sum is at least 1 in
    # final units, so the error of O is at most sum_j (p_j / 16 + 2^-10 / c) |v_j|
    g = torch.Generator().manual_seed(408)
    B, N, H, d = 1, 40, 2, 16
    q8 = torch.randint(0, 255, (B, N, H, d), generator=g).to(torch.uint8)
    k8 = torch.randint(0, 255, (B, N, H, d), generator=g).to(torch.uint8)
    v8 = torch.randint(0, 255, (B, N, H, d), generator=g).to(torch.uint8)
    for t in (q8, k8, v8):
        t[(t & 127) == 127] = 0x38                     # no NaN codes
    # one scale per block of 16 rows, different in every block, head and tensor
    sq = torch.ldexp(torch.ones(B, H, 3, dtype=torch.float64), torch.tensor([[[-6., -4., -7.], [-5., -6., -8.]]]))
    sk = torch.ldexp(torch.ones(B, H, 3, dtype=torch.float64), torch.tensor([[[-5., -7., -6.], [-4., -5., -7.]]]))
    sv = torch.ldexp(torch.ones(B, H, 3, dtype=torch.float64), torch.tensor([[[-3., -1., -4.], [-2., -5., -3.]]]))

    def rows(sc):   # the scale of each row, [B, N, H, 1]
        return sc.repeat_interleave(16, dim=2)[:, :, :N].transpose(1, 2)[..., None]

    for causal, tau in ((False, 0.0), (True, 0.0), (False, f.RESCALE_LOG2), (True, f.RESCALE_LOG2)):
        o, lse, _, _ = f.fp8_attention_forward(q8, k8, v8, sq, sk, sv, 0.37, causal, scale_rows=16,
                                               block=8, rescale_log2=tau)
        qd = f.e4m3_decode(q8) * rows(sq)
        kd = f.e4m3_decode(k8) * rows(sk)
        vd = f.e4m3_decode(v8) * rows(sv)
        o_ref, lse_ref = dense.attention_forward(qd, kd, vd, 0.37, causal)
        p = dense.attention_probs(qd, kd, 0.37, causal)            # [B, H, N, N]
        bound = torch.einsum("bhij,bjhd->bihd", p / 16 + 2.0 ** -10 / 2.0 ** (8 - tau), vd.abs())
        diff = (o - o_ref).abs()
        assert bool((diff <= bound * (1 + 1e-9) + 1e-13).all()), (causal, tau)
        assert diff.max().item() > 1e-6                            # P~ is rounded
        assert (lse - lse_ref).abs().max().item() < 1e-10


def pin_fp8_slack_covers_p_rounding(f):
    # with every P code counted as near a tie (p_tie_rel = 1) and exact Q, K, V,
    # slack_o is sum_j step(p8_j) |v_j| in the row's final units, which bounds
    # the effect of rounding P: |O - O_exact| <= slack_o + sum_j 2^-10 / c |v_j|
    # (c = 2^(8 - tau); the second term: subnormal codes, rounded by less than
    # 2^-10 / c but too small to count as near a tie).  Random codes in blocks
    # of 8 keys give rows whose reference stays below the true maximum.
    g = torch.Generator().manual_seed(413)
    B, N, H, d = 1, 96, 2, 16
    q8, k8, v8 = (torch.randint(0, 255, (B, N, H, d), generator=g).to(torch.uint8) for _ in range(3))
    for t in (q8, k8, v8):
        t[(t & 127) >= 0x70] = 0x30                    # no NaN codes, magnitudes below 2^7
    ones = torch.ones(B, H, 2, dtype=torch.float64)
    qd, kd, vd = f.e4m3_decode(q8), f.e4m3_decode(k8), f.e4m3_decode(v8)
    for causal in (False, True):
        o, lse, so, _ = f.fp8_attention_forward(q8, k8, v8, ones, ones, ones, 2e-4, causal, p_tie_rel=1.0,
                                                block=8)
        assert bool(torch.isfinite(so).all())
        o_ref, _ = dense.attention_forward(qd, kd, vd, 2e-4, causal)
        tol = 2.0 ** -10 / 2.0 ** (8 - f.RESCALE_LOG2) * vd.abs().sum(dim=1, keepdim=True)
        assert bool(((o - o_ref).abs() <= so * (1 + 1e-9) + tol + 1e-13).all()), causal


def pin_fp8_forward_close_and_rotation_helps(f):
    B, N, H, d = 1, 96, 2, 64
    q, k, v = _rand((B, N, H, d), 409), _rand((B, N, H, d), 410), _rand((B, N, H, d), 411)
    sg = _signs(d, 412)
    scale = d ** -0.5
    o_ref, lse_ref = dense.attention_forward(q, k, v, scale, False)
    o_rot = f.fp8_forward(q, k, v, sg, scale, False, rotate_qk=True)[0]
    assert f.rmse(o_rot, o_ref) < 3e-2
    # outliers: two channels of Q and K twenty times larger
    qo, ko = q.clone(), k.clone()
    qo[..., [5, 40]] *= 20.0
    ko[..., [5, 40]] *= 20.0
    scale_o = 0.02
    o_ref2, _ = dense.attention_forward(qo, ko, v, scale_o, False)
    e_plain = f.rmse(f.fp8_forward(qo, ko, v, sg, scale_o, False, rotate_qk=False)[0], o_ref2)
    e_rot = f.rmse(f.fp8_forward(qo, ko, v, sg, scale_o, False, rotate_qk=True)[0], o_ref2)
    assert e_rot < e_plain, (e_rot, e_plain)


def _fwht32(x):
    """Fast Walsh-Hadamard transform along the last axis in float32 (butterflies
    of stride 1, 2, 4, ...: each stage rounds once), the transform the page's
    rotation needs, computed the way a GPU computes it."""
    d = x.shape[-1]
    y = x.to(torch.float32)
    h = 1
    while h < d:
        y = y.reshape(*x.shape[:-1], d // (2 * h), 2, h)
        a, b = y[..., 0, :], y[..., 1, :]
        y = torch.stack([a + b, a - b], dim=-2).reshape(*x.shape[:-1], d)
        h *= 2
    return y.to(torch.float64)


def pin_fp8_rotation_error_bound(f):
    # the bound on |fp32 rotation - exact| / s holds for every element of random
    # rows and of rows whose partial sums keep growing (x_i = sigma_i (1 + u_i 2^-6),
    # so every butterfly adds like-signed terms), and on the latter it is within a
    # factor 5 of the worst element of some row (not a loose bound that any
    # rotation error passes); a different power-of-two scale in each 64-row block
    d = 128
    g = torch.Generator().manual_seed(414)
    sg = (torch.randint(0, 2, (d,), generator=g) * 2 - 1).to(torch.float64)
    rnd = torch.randn(1, 256, 1, d, generator=g, dtype=torch.float32).to(torch.float64)
    u = torch.rand(1, 256, 1, d, generator=g, dtype=torch.float32).to(torch.float64)
    coh = (sg * (1 + u * 2.0 ** -6)).to(torch.float32).to(torch.float64)
    s = torch.tensor([[[0.125, 0.25, 0.0625, 0.5]]], dtype=torch.float64)
    rows = s.repeat_interleave(64, dim=2).transpose(1, 2)[..., None]          # [1, 256, 1, 1]
    for x, tight in ((rnd, False), (coh, True)):
        err = (_fwht32(x * sg) - f.rotate(x, sg)).abs() / rows
        bnd = f.fp32_rotation_error(x, sg, s)
        assert bnd.shape == (1, 256, 1, 1)
        assert bool((err <= bnd).all())
        if tight:
            assert (bnd / err.amax(-1, keepdim=True)).min().item() <= 5.0


def _vec(vals):
    """[1, n, 1, 4] with the first component of each row set (exact e4m3 values
    or pre-rounding values)."""
    t = torch.zeros(1, len(vals), 1, 4, dtype=torch.float64)
    t[0, :, 0, 0] = torch.tensor([float(v) for v in vals], dtype=torch.float64)
    return t


def _flip_bounds(d_o, d_l, so, sl, what, ds=0.0):
    """One near-tie code rounded the other way moves O by d_o and LSE by d_l: the
    slack covers that move and is at most 1.5 times it (not inflated).  The
    slack is a first-order bound: a flip that moves a score by ds leaves a
    second-order remainder of relative size at most about ds, allowed here."""
    so, sl = float(so), float(sl)
    allow = 1.0 + ds + 1e-6
    assert d_o <= allow * so + 1e-12, (what, d_o, so)
    assert so <= 1.5 * d_o + 1e-12, (what, d_o, so)
    if d_l > 1e-9:
        assert d_l <= allow * sl + 1e-12 and sl <= 1.5 * d_l, (what, d_l, sl)
    else:
        assert sl == 0.0, (what, sl)


def pin_fp8_tie_slack_single_flip(f):
    # one query, two keys, values only in component 0; exactly one code of each
    # kind sits at a near-tie (within 1e-7 relative of a midpoint).  For P and V
    # the oracle's own output with the code rounded each way is compared (P,
    # through a score scale just below / above the tie); for Q and K, whose flip
    # also re-rounds the probabilities, the exact dense attention on the decoded
    # inputs with either code (the slack bounds the score effect, to first order)
    enc, dec = f.e4m3_encode, f.e4m3_decode
    one = torch.ones(1, 1, dtype=torch.float64)
    # P: keys 2, 1 (q = 1), scores 2c, c; 16 exp(-c) = 12.5 is the midpoint of the
    # codes 12 and 13, so P~_1 rounds to 12 or 13 as c crosses c0; values 1, 3
    q8, k8, v8 = enc(_vec([1.0])), enc(_vec([2.0, 1.0])), enc(_vec([1.0, 3.0]))
    c0 = math.log(16.0 / 12.5)
    res = [f.fp8_attention_forward(q8, k8, v8, one, one, one, c, False, block=None)
           for c in (c0 * (1 + 1e-9), c0 * (1 - 1e-9))]
    assert f.RESCALE_LOG2 == 4.0
    _flip_bounds((res[1][0] - res[0][0]).abs()[0, 0, 0, 0].item(),
                 (res[1][1] - res[0][1]).abs().item(), res[0][2][0, 0, 0, 0], res[0][3][0, 0, 0], "P")
    assert res[0][2][0, 0, 0, 1:].abs().max().item() == 0.0
    # V: scores 0, -ln 2 give exact P~ 1, 1/2; v_1 = 2.625 (1 + 1e-7) lies at the
    # midpoint of 2.5 and 2.75 (in units of V's scale, 0.5)
    vs = _vec([-2.0, 2.625 * (1 + 1e-7)])
    q8, k8 = enc(_vec([1.0])), enc(_vec([0.0, -1.0]))
    v8, v8alt = enc(vs), enc(_vec([-2.0, 2.5]))
    assert dec(v8)[0, 1, 0, 0].item() == 2.75
    sv = one * 0.5                                    # V in units of its scale
    o, lse, so, sl = f.fp8_attention_forward(q8, k8, v8, one, one, sv, math.log(2.0), False,
                                             v_scaled=vs, block=None)
    oa, lsea, _, _ = f.fp8_attention_forward(q8, k8, v8alt, one, one, sv, math.log(2.0), False, block=None)
    _flip_bounds((oa - o).abs()[0, 0, 0, 0].item(), (lsea - lse).abs().item(), so[0, 0, 0, 0], sl[0, 0, 0], "V")
    # Q: q_0 = 1.0625 (1 + 1e-7), the midpoint of 1 and 1.125; keys 0, -1 (so only
    # the second score moves), values -2, 3 (on either side of O = -1, so the first-
    # order bound is tight)
    qs, ks, vs = _vec([1.0625 * (1 + 1e-7)]), _vec([0.0, -1.0]), _vec([-2.0, 3.0])
    q8, q8alt, k8, v8 = enc(qs), enc(_vec([1.0])), enc(ks), enc(vs)
    o, lse, so, sl = f.fp8_attention_forward(q8, k8, v8, one, one, one, 1.25, False, q_scaled=qs,
                                             k_scaled=ks, block=None, p_tie_rel=0.0)
    e0 = dense.attention_forward(dec(q8), dec(k8), dec(v8), 1.25, False)
    e1 = dense.attention_forward(dec(q8alt), dec(k8), dec(v8), 1.25, False)
    _flip_bounds((e1[0] - e0[0]).abs()[0, 0, 0, 0].item(), (e1[1] - e0[1]).abs().item(),
                 so[0, 0, 0, 0], sl[0, 0, 0], "Q", ds=1.25 * 0.125)
    # K: q = -1, k_1 = 1.0625 (1 + 1e-7), the same midpoint
    qs, ks = _vec([-1.0]), _vec([0.0, 1.0625 * (1 + 1e-7)])
    q8, k8, k8alt = enc(qs), enc(ks), enc(_vec([0.0, 1.0]))
    o, lse, so, sl = f.fp8_attention_forward(q8, k8, v8, one, one, one, 1.25, False, q_scaled=qs,
                                             k_scaled=ks, block=None, p_tie_rel=0.0)
    e0 = dense.attention_forward(dec(q8), dec(k8), dec(v8), 1.25, False)
    e1 = dense.attention_forward(dec(q8), dec(k8alt), dec(v8), 1.25, False)
    _flip_bounds((e1[0] - e0[0]).abs()[0, 0, 0, 0].item(), (e1[1] - e0[1]).abs().item(),
                 so[0, 0, 0, 0], sl[0, 0, 0], "K", ds=1.25 * 0.125)


ALL_PINS = [
    pin_e4m3_named_codes,
    pin_e4m3_encode_is_nearest,
    pin_hadamard,
    pin_rotation_keeps_scores,
    pin_quantize_scale_and_codes,
    pin_fp8_attention_exact_powers_of_two,
    pin_fp8_running_max_worked_example,
    pin_fp8_conditional_rescale_worked_example,
    pin_fp8_rescale_near_tie_flagged,
    pin_fp8_attention_p_rounding_bound,
    pin_fp8_slack_covers_p_rounding,
    pin_fp8_forward_close_and_rotation_helps,
    pin_fp8_rotation_error_bound,
    pin_fp8_tie_slack_single_flip,
]
