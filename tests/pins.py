"""Checks that tie the CPU oracle to facts fixed outside the oracle itself.

Each ``pin_*`` function takes an oracle module (normally ``oracle``; the
mutation tests pass copies with a planted mistake) and raises AssertionError
when the oracle disagrees with the fact it checks.  The facts come from the
pages' definition of attention and from mathematics:

* rows of P sum to one (definition of softmax, "08 · FlashAttention", §二);
* the online update over any key-block split equals the one-shot result
  ("08 · FlashAttention", §二; "LLM Systems 22: Flash Attention", §3.1);
* special cases with closed forms (identical keys, one dominating score,
  causal row 0), shift and permutation invariance (the exponent identity of
  "LLM Systems 22: Flash Attention", §3.1);
* torch-CPU float64 ``scaled_dot_product_attention`` and ``torch.logsumexp``
  (the library routine "08 · FlashAttention", §四 names), with autograd for
  the gradients;
* central finite differences and gradient invariants.
"""

from __future__ import annotations

import math
import random

import torch
import torch.nn.functional as F


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64) * scale


def _sdpa(q, k, v, scale, causal):
    """torch fp64 SDPA on [B, N, H, d] tensors (it wants [B, H, N, d])."""
    qt, kt, vt = (x.transpose(1, 2) for x in (q, k, v))
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
    return o.transpose(1, 2)


def _lse_lib(q, k, scale, causal):
    s = scale * torch.einsum("bihd,bjhd->bhij", q, k)
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    return torch.logsumexp(s, dim=-1)


def pin_row_sums(orc):
    for causal in (False, True):
        q, k = _rand((2, 37, 3, 16), 1, 3.0), _rand((2, 37, 3, 16), 2, 3.0)
        p = orc.attention_probs(q, k, 0.37, causal)
        err = (p.sum(-1) - 1.0).abs().max().item()
        assert err < 1e-14, f"row sums off by {err} (causal={causal})"
        assert (p >= 0).all()
        if causal:
            assert (p.triu(1) == 0).all(), "causal P has weight above the diagonal"


def pin_online_equals_oneshot(orc):
    rnd = random.Random(7)
    for causal in (False, True):
        B, N, H, d = 2, 53, 2, 8
        q, k, v = _rand((B, N, H, d), 11), _rand((B, N, H, d), 12), _rand((B, N, H, d), 13)
        # make the running max rise and fall across blocks
        k[:, ::7] *= 4.0
        k[:, 3::11] *= -3.0
        o_ref, lse_ref = orc.attention_forward(q, k, v, 0.5, causal)
        for trial in range(6):
            cuts = sorted(rnd.sample(range(1, N), rnd.randint(1, 12)))
            if trial == 0:
                cuts = list(range(1, N))          # blocks of one key
            bnd = [0] + cuts + [N]
            o, lse = orc.online_softmax_forward(q, k, v, 0.5, causal, bnd)
            eo = (o - o_ref).abs().max().item()
            el = (lse - lse_ref).abs().max().item()
            assert eo < 1e-12 and el < 1e-12, f"online vs one-shot: O {eo}, LSE {el} ({bnd})"


def pin_uniform_keys(orc):
    B, N, H, d = 1, 19, 2, 6
    q, v = _rand((B, N, H, d), 21), _rand((B, N, H, d), 22)
    key = _rand((1, 1, H, d), 23)
    k = key.expand(B, N, H, d).clone()
    scale = 0.8
    s = scale * torch.einsum("bihd,bjhd->bhi", q, key)        # the single score per row
    o, lse = orc.attention_forward(q, k, v, scale, False)
    mean_v = v.mean(dim=1, keepdim=True).expand_as(o)
    assert (o - mean_v).abs().max().item() < 1e-13
    assert (lse - (s + math.log(N))).abs().max().item() < 1e-12
    o, lse = orc.attention_forward(q, k, v, scale, True)
    cnt = torch.arange(1, N + 1, dtype=torch.float64)
    run_mean = v.cumsum(dim=1) / cnt.view(1, N, 1, 1)
    assert (o - run_mean).abs().max().item() < 1e-13
    assert (lse - (s + torch.log(cnt).view(1, 1, N))).abs().max().item() < 1e-12


def pin_one_hot(orc):
    B, N, H, d = 1, 24, 1, 8
    k = _rand((B, N, H, d), 31)
    v = _rand((B, N, H, d), 32)
    target = 13
    q = torch.zeros(B, N, H, d, dtype=torch.float64)
    # each query points along key `target`, scaled so that score gap >= 40
    kt = k[0, target, 0]
    others = torch.cat([k[0, :target, 0], k[0, target + 1:, 0]])
    gap_per_unit = (kt @ kt - (others @ kt).max()).item()
    assert gap_per_unit > 0
    q[0, :, 0] = kt * (60.0 / gap_per_unit)
    o, lse = orc.attention_forward(q, k, v, 1.0, False)
    bound = v.abs().max().item() * N * math.exp(-40.0)
    assert (o[0, :, 0] - v[0, target, 0]).abs().max().item() <= bound + 1e-15
    s_t = (q[0, :, 0] @ kt)
    assert (lse[0, 0] - s_t).abs().max().item() <= N * math.exp(-40.0) + 1e-12


def pin_shift_invariance(orc):
    B, N, H, d = 1, 29, 2, 8
    q, k, v = _rand((B, N, H, d), 41), _rand((B, N, H, d), 42), _rand((B, N, H, d), 43)
    scale = 0.7
    for mag in (1.0, 1000.0):
        u = _rand((1, 1, H, d), 44) * mag
        for causal in (False, True):
            o0, l0 = orc.attention_forward(q, k, v, scale, causal)
            o1, l1 = orc.attention_forward(q, k + u, v, scale, causal)
            qu = scale * torch.einsum("bihd,bjhd->bhi", q, u)
            assert torch.isfinite(o1).all() and torch.isfinite(l1).all(), "overflow under key shift"
            assert (o1 - o0).abs().max().item() < 1e-9 * max(1.0, mag)
            assert ((l1 - l0 - qu).abs() / (1 + qu.abs())).max().item() < 1e-12


def pin_permutation(orc):
    B, N, H, d = 2, 23, 2, 8
    q, k, v = _rand((B, N, H, d), 51), _rand((B, N, H, d), 52), _rand((B, N, H, d), 53)
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(54))
    o0, l0 = orc.attention_forward(q, k, v, 0.9, False)
    o1, l1 = orc.attention_forward(q, k[:, perm], v[:, perm], 0.9, False)
    assert (o1 - o0).abs().max().item() < 1e-13
    assert (l1 - l0).abs().max().item() < 1e-13


def pin_causal_row0(orc):
    B, N, H, d = 2, 17, 3, 8
    q, k, v = _rand((B, N, H, d), 61), _rand((B, N, H, d), 62), _rand((B, N, H, d), 63)
    scale = 1.3
    o, lse = orc.attention_forward(q, k, v, scale, True)
    assert (o[:, 0] == v[:, 0]).all(), "causal row 0 must equal V row 0 exactly"
    s00 = scale * (q[:, 0] * k[:, 0]).sum(-1)          # [B, H]
    assert (lse[:, :, 0] - s00).abs().max().item() < 1e-14


def pin_library_forward(orc):
    for causal in (False, True):
        for (B, N, H, d, scale) in ((2, 40, 3, 16, 0.25), (1, 65, 2, 64, 0.125), (1, 33, 1, 8, 2.0)):
            q, k, v = _rand((B, N, H, d), 71), _rand((B, N, H, d), 72), _rand((B, N, H, d), 73)
            o, lse = orc.attention_forward(q, k, v, scale, causal, row_chunk=16)
            o_ref = _sdpa(q, k, v, scale, causal)
            l_ref = _lse_lib(q, k, scale, causal)
            assert (o - o_ref).abs().max().item() < 1e-12, "O differs from torch SDPA"
            assert (lse - l_ref).abs().max().item() < 1e-12, "LSE differs from torch.logsumexp"
    # non-square, non-causal
    q, k, v = _rand((2, 21, 2, 8), 74), _rand((2, 34, 2, 8), 75), _rand((2, 34, 2, 8), 76)
    o, _ = orc.attention_forward(q, k, v, 0.3, False)
    assert (o - _sdpa(q, k, v, 0.3, False)).abs().max().item() < 1e-12


def pin_library_backward(orc):
    for causal in (False, True):
        for (B, N, H, d, scale) in ((2, 40, 3, 16, 0.25), (1, 47, 2, 32, 0.6)):
            q, k, v = (_rand((B, N, H, d), s).requires_grad_() for s in (81, 82, 83))
            do = _rand((B, N, H, d), 84)
            o_ref = _sdpa(q, k, v, scale, causal)
            gq, gk, gv = torch.autograd.grad(o_ref, (q, k, v), do)
            dq, dk, dv, _ = orc.attention_backward(q, k, v, do, scale, causal, row_chunk=16)
            for name, a, b in (("dq", dq, gq), ("dk", dk, gk), ("dv", dv, gv)):
                err = (a - b).abs().max().item()
                assert err < 1e-11, f"{name} differs from autograd by {err} (causal={causal})"


def pin_finite_differences(orc):
    for causal in (False, True):
        B, N, H, d, scale = 1, 6, 1, 4, 0.9
        q, k, v, do = (_rand((B, N, H, d), s) for s in (91, 92, 93, 94))
        dq, dk, dv, _ = orc.attention_backward(q, k, v, do, scale, causal)

        def loss(qq, kk, vv):
            return (orc.attention_forward(qq, kk, vv, scale, causal)[0] * do).sum().item()

        h = 1e-6
        for which, g in ((0, dq), (1, dk), (2, dv)):
            for idx in range(q.numel()):
                args = [q.clone(), k.clone(), v.clone()]
                flat = args[which].view(-1)
                flat[idx] += h
                lp = loss(*args)
                flat[idx] -= 2 * h
                lm = loss(*args)
                fd = (lp - lm) / (2 * h)
                an = g.reshape(-1)[idx].item()
                assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), \
                    f"finite difference {fd} vs analytic {an} (tensor {which}, idx {idx}, causal={causal})"


def pin_gradient_invariants(orc):
    for causal in (False, True):
        B, N, H, d = 2, 31, 2, 16
        q, k, v, do = (_rand((B, N, H, d), s) for s in (101, 102, 103, 104))
        dq, dk, dv, dvec = orc.attention_backward(q, k, v, do, 0.4, causal, row_chunk=8)
        o, _ = orc.attention_forward(q, k, v, 0.4, causal)
        # a common shift of all keys leaves softmax unchanged -> sum_j dK_j = 0
        assert dk.sum(dim=1).abs().max().item() < 1e-12
        # rows of P sum to one -> sum_j dV_j = sum_i dO_i
        assert (dv.sum(dim=1) - do.sum(dim=1)).abs().max().item() < 1e-12
        # D = rowsum(P * dP) = rowsum(dO * O)
        d_alt = (do * o).sum(-1).transpose(1, 2)
        assert (dvec - d_alt).abs().max().item() < 1e-12


def pin_varlen(orc):
    lengths = [5, 1, 17, 0, 9]
    H, d, scale = 2, 8, 0.35
    total = sum(lengths)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    q, k, v, do = (_rand((total, H, d), s) for s in (111, 112, 113, 114))
    for causal in (False, True):
        o, lse = orc.attention_forward_varlen(q, k, v, cu, cu, max(lengths), scale, causal)
        dq, dk, dv = orc.attention_backward_varlen(q, k, v, do, cu, cu, scale, causal)
        for s, n in enumerate(lengths):
            if n == 0:
                assert torch.isnan(lse[s]).all()
                continue
            sl = slice(cu[s], cu[s + 1])
            qs, ks, vs = (x[None, sl].clone().requires_grad_() for x in (q, k, v))
            o_ref = _sdpa(qs, ks, vs, scale, causal)
            assert (o[sl] - o_ref[0]).abs().max().item() < 1e-12
            l_ref = _lse_lib(qs.detach(), ks.detach(), scale, causal)[0]
            assert (lse[s, :, :n] - l_ref).abs().max().item() < 1e-12
            assert torch.isnan(lse[s, :, n:]).all()
            g = torch.autograd.grad(o_ref, (qs, ks, vs), do[None, sl])
            for a, b in ((dq[sl], g[0][0]), (dk[sl], g[1][0]), (dv[sl], g[2][0])):
                assert (a - b).abs().max().item() < 1e-11
    # non-causal with key lengths that differ from the query lengths
    klens = [3, 4, 11, 2, 9]
    cuk = [0]
    for n in klens:
        cuk.append(cuk[-1] + n)
    k2, v2 = _rand((cuk[-1], H, d), 115), _rand((cuk[-1], H, d), 116)
    o, lse = orc.attention_forward_varlen(q, k2, v2, cu, cuk, max(lengths), scale, False)
    dq, dk, dv = orc.attention_backward_varlen(q, k2, v2, do, cu, cuk, scale, False)
    for s, n in enumerate(lengths):
        if n == 0:
            continue
        sq, sk = slice(cu[s], cu[s + 1]), slice(cuk[s], cuk[s + 1])
        qs = q[None, sq].clone().requires_grad_()
        ks, vs = (x[None, sk].clone().requires_grad_() for x in (k2, v2))
        o_ref = _sdpa(qs, ks, vs, scale, False)
        assert (o[sq] - o_ref[0]).abs().max().item() < 1e-12
        g = torch.autograd.grad(o_ref, (qs, ks, vs), do[None, sq])
        for a, b in ((dq[sq], g[0][0]), (dk[sk], g[1][0]), (dv[sk], g[2][0])):
            assert (a - b).abs().max().item() < 1e-11


ALL_PINS = [
    pin_row_sums,
    pin_online_equals_oneshot,
    pin_uniform_keys,
    pin_one_hot,
    pin_shift_invariance,
    pin_permutation,
    pin_causal_row0,
    pin_library_forward,
    pin_library_backward,
    pin_finite_differences,
    pin_gradient_invariants,
    pin_varlen,
]
