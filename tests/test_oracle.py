"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each pin is a function of the oracle module so that the planted-mistake tests
at the end can run the same pins against deliberately broken copies of the
oracle (on the CPU) and show that every such mistake fails at least one pin.

Pins (what each one fixes):
* closed form 2x2 fixture (hand-derived; tests/golden/closed_form_2x2.json)
* rows of P sum to one (softmax definition)
* constant keys: O is the mean of the visible V rows, LSE = scale q.k + ln(#visible)
* a dominant score selects one V row
* causal row 0 returns V[0]; N = 1 returns V
* key-shift and key/value-permutation invariance
* tiled online softmax (Eq. (1)-(2) of the Journal of Software survey) and the
  two-pass tiled softmax equal the direct result on tiny inputs
* torch's CPU float64 scaled_dot_product_attention and logsumexp (library routine)
* gradients: central finite differences, torch.autograd on plain fp64 ops,
  and the invariants sum_j dK_j = 0, sum_j dV_j = sum_i dO_i, constant keys => dQ = 0
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.ref as ref_module
from oracle import online_softmax as osm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_2x2.json")


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).normal(0.0, std, size=shape)


# ----------------------------------------------------------------------------
# pin functions: each takes the oracle module R and raises AssertionError
# ----------------------------------------------------------------------------

def pin_golden(R):
    g = json.load(open(GOLDEN))
    q, k, v, do = (np.array(g[n])[None, None] for n in ("q", "k", "v", "do"))
    for mode, causal in (("noncausal", False), ("causal", True)):
        exp = g[mode]
        o, lse = R.ref_fwd(q, k, v, g["scale"], causal)
        np.testing.assert_allclose(o[0, 0], exp["o"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, 0], exp["lse"], rtol=0, atol=1e-14)
        dq, dk, dv = R.ref_bwd(q, k, v, do, g["scale"], causal)
        np.testing.assert_allclose(dq[0, 0], exp["dq"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(dk[0, 0], exp["dk"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(dv[0, 0], exp["dv"], rtol=0, atol=1e-14)


def pin_rows_sum_to_one(R):
    q, k = _rand((2, 2, 37, 16), 1), _rand((2, 2, 37, 16), 2, 3.0)
    for causal in (False, True):
        p = R.ref_probs(q, k, 0.25, causal)
        assert np.all(p >= 0)
        np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-14)
        if causal:
            assert np.all(np.triu(p[0, 0], k=1) == 0)
            assert np.all(np.diagonal(p[0, 0]) > 0)


def pin_constant_keys(R):
    B, H, N, d = 1, 2, 23, 8
    q, v = _rand((B, H, N, d), 3), _rand((B, H, N, d), 4)
    kvec = _rand((B, H, 1, d), 5)
    k = np.repeat(kvec, N, axis=2)
    scale = 0.3
    for causal in (False, True):
        o, lse = R.ref_fwd(q, k, v, scale, causal)
        for h in range(H):
            for i in range(N):
                nvis = i + 1 if causal else N
                np.testing.assert_allclose(o[0, h, i], v[0, h, :nvis].mean(0), rtol=0, atol=1e-13)
                want = scale * float(q[0, h, i] @ kvec[0, h, 0]) + math.log(nvis)
                assert abs(lse[0, h, i] - want) < 1e-13


def pin_dominant_score(R):
    N, d = 19, 6
    q, k, v = _rand((1, 1, N, d), 6), _rand((1, 1, N, d), 7), _rand((1, 1, N, d), 8)
    i, t = 11, 4
    k[0, 0, t] = 40.0 * q[0, 0, i] / np.linalg.norm(q[0, 0, i])
    s = k[0, 0] @ q[0, 0, i]
    assert s[t] - np.max(np.delete(s, t)) >= 50
    o, _ = R.ref_fwd(q, k, v, 1.0, False)
    np.testing.assert_allclose(o[0, 0, i], v[0, 0, t], rtol=0, atol=N * math.exp(-50) * 10)


def pin_causal_row0_and_n1(R):
    q, k, v = _rand((2, 3, 17, 8), 9), _rand((2, 3, 17, 8), 10), _rand((2, 3, 17, 8), 11)
    o, lse = R.ref_fwd(q, k, v, 0.35, True)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[:, :, 0], 0.35 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               rtol=0, atol=1e-14)
    for causal in (False, True):
        o1, lse1 = R.ref_fwd(q[:, :, :1], k[:, :, :1], v[:, :, :1], 0.35, causal)
        np.testing.assert_allclose(o1, v[:, :, :1], rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse1[..., 0], 0.35 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                                   rtol=0, atol=1e-14)


def pin_shift_and_permutation(R):
    N, d = 21, 8
    q, k, v = _rand((1, 2, N, d), 12), _rand((1, 2, N, d), 13), _rand((1, 2, N, d), 14)
    c = _rand((1, 2, 1, d), 15)
    scale = 0.4
    for causal in (False, True):
        o, lse = R.ref_fwd(q, k, v, scale, causal)
        o2, lse2 = R.ref_fwd(q, k + c, v, scale, causal)
        np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse2 - lse, scale * np.einsum("bhnd,bhd->bhn", q, c[:, :, 0]),
                                   rtol=0, atol=1e-12)
    perm = np.random.default_rng(16).permutation(N)
    o, lse = R.ref_fwd(q, k, v, scale, False)
    o3, lse3 = R.ref_fwd(q, k[:, :, perm], v[:, :, perm], scale, False)
    np.testing.assert_allclose(o3, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse3, lse, rtol=0, atol=1e-12)


def pin_tiled_equals_direct(R):
    for (N, d, seed) in ((16, 8, 20), (13, 5, 21), (7, 3, 22)):
        q, k, v = _rand((1, 1, N, d), seed, 2.0), _rand((1, 1, N, d), seed + 1, 2.0), _rand((1, 1, N, d), seed + 2)
        for causal in (False, True):
            o, lse = R.ref_fwd(q, k, v, 0.5, causal)
            for bq, bk in ((1, 1), (2, 3), (3, 5), (5, 2), (N, N), (4, N)):
                ot, lt = osm.tiled_attention_fwd(q, k, v, 0.5, causal, bq, bk)
                np.testing.assert_allclose(ot, o, rtol=0, atol=1e-12)
                np.testing.assert_allclose(lt, lse, rtol=0, atol=1e-12)
    # the two block-softmax variants of the pages on single vectors
    qv, kv = _rand((1, 1, 11, 4), 30), _rand((1, 1, 11, 4), 31, 3.0)
    p = R.ref_probs(qv, kv, 1.0, False)[0, 0, 5]
    x = kv[0, 0] @ qv[0, 0, 5]
    for blk in (1, 2, 3, 5, 11):
        np.testing.assert_allclose(osm.online_softmax(x, blk), p, rtol=0, atol=1e-15)
        np.testing.assert_allclose(osm.two_pass_softmax(x, blk), p, rtol=0, atol=1e-15)


def pin_torch_sdpa(R):
    B, H, N, d = 2, 3, 45, 16
    q, k, v = _rand((B, H, N, d), 40), _rand((B, H, N, d), 41, 2.0), _rand((B, H, N, d), 42)
    scale = 0.2
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    for causal in (False, True):
        o, lse = R.ref_fwd(q, k, v, scale, causal)
        to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
        np.testing.assert_allclose(o, to.numpy(), rtol=0, atol=1e-13)
        s = scale * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
        np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-13)
        rows = [0, 1, 7, 44, 20]
        orow, lrow = R.ref_fwd_rows(q[1, 2], k[1, 2], v[1, 2], scale, causal, rows)
        np.testing.assert_allclose(orow, to.numpy()[1, 2, rows], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lrow, torch.logsumexp(s, -1).numpy()[1, 2, rows], rtol=0, atol=1e-13)


def _loss(R, q, k, v, do, scale, causal):
    return float((R.ref_fwd(q, k, v, scale, causal)[0] * do).sum())


def pin_finite_differences(R):
    N, d, scale, eps = 6, 4, 0.7, 1e-6
    q, k, v, do = (_rand((1, 1, N, d), 50 + i) for i in range(4))
    for causal in (False, True):
        grads = R.ref_bwd(q, k, v, do, scale, causal)
        for which, g in enumerate(grads):
            num = np.zeros_like(g)
            for idx in np.ndindex(*g.shape):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][idx] += eps
                lp = _loss(R, *args, do, scale, causal)
                args[which][idx] -= 2 * eps
                lm = _loss(R, *args, do, scale, causal)
                num[idx] = (lp - lm) / (2 * eps)
            np.testing.assert_allclose(g, num, rtol=1e-7, atol=1e-8)


def pin_autograd(R):
    B, H, N, d = 1, 2, 11, 5
    arrs = [_rand((B, H, N, d), 60 + i) for i in range(4)]
    scale = 0.45
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in arrs[:3])
        s = scale * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
        o = torch.softmax(s, -1) @ tv
        (o * torch.from_numpy(arrs[3])).sum().backward()
        dq, dk, dv = R.ref_bwd(*arrs, scale, causal)
        np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-13)
        np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-13)


def pin_bwd_rows(R):
    """The row-subset backward against torch autograd (fp64, CPU) of sum(O * dO) with dO
    zeroed outside the rows: dQ of the rows, and the rows' whole contribution to dK, dV."""
    B, H, N, d = 1, 1, 23, 6
    arrs = [_rand((B, H, N, d), 70 + i, 1.5) for i in range(4)]
    scale = 0.35
    cases = [([0, 3, 22, 11], [0, 5, 22], False), ([2, 19, 20, 21, 22], [19, 20, 21, 22], True),
             (list(range(N)), list(range(N)), True)]
    for rows, keys, causal in cases:
        tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in arrs[:3])
        s = scale * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
        o = torch.softmax(s, -1) @ tv
        dmask = np.zeros_like(arrs[3])
        dmask[0, 0, rows] = arrs[3][0, 0, rows]
        (o * torch.from_numpy(dmask)).sum().backward()
        dq, dk, dv = R.ref_bwd_rows(arrs[0][0, 0], arrs[1][0, 0], arrs[2][0, 0], arrs[3][0, 0], scale, causal,
                                    rows, keys)
        np.testing.assert_allclose(dq, tq.grad.numpy()[0, 0, rows], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dk, tk.grad.numpy()[0, 0, keys], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv, tv.grad.numpy()[0, 0, keys], rtol=0, atol=1e-13)


def pin_gradient_invariants(R):
    B, H, N, d = 1, 2, 19, 8
    q, k, v, do = (_rand((B, H, N, d), 70 + i) for i in range(4))
    for causal in (False, True):
        dq, dk, dv = R.ref_bwd(q, k, v, do, 0.3, causal)
        np.testing.assert_allclose(dk.sum(2), 0.0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv.sum(2), do.sum(2), rtol=0, atol=1e-12)
        kc = np.repeat(k[:, :, :1], N, axis=2)
        dqc, _, _ = R.ref_bwd(q, kc, v, do, 0.3, causal)
        np.testing.assert_allclose(dqc, 0.0, rtol=0, atol=1e-12)
        # D from (O, dO) equals rowsum(P * dP)
        o, _ = R.ref_fwd(q, k, v, 0.3, causal)
        p = R.ref_probs(q, k, 0.3, causal)
        dp = do @ v.transpose(0, 1, 3, 2)
        np.testing.assert_allclose(R.ref_bwd_delta(o, do), (p * dp).sum(-1), rtol=0, atol=1e-12)


def pin_large_spread(R):
    """Scores of magnitude ~1e3 must not overflow (the max is subtracted before exp)."""
    N, d = 9, 4
    q, k, v = _rand((1, 1, N, d), 80, 30.0), _rand((1, 1, N, d), 81, 30.0), _rand((1, 1, N, d), 82)
    for causal in (False, True):
        o, lse = R.ref_fwd(q, k, v, 1.0, causal)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        ot, lt = osm.tiled_attention_fwd(q, k, v, 1.0, causal, 2, 3)
        np.testing.assert_allclose(o, ot, rtol=0, atol=1e-10)
        np.testing.assert_allclose(lse, lt, rtol=1e-14, atol=1e-9)


PINS = [pin_golden, pin_rows_sum_to_one, pin_constant_keys, pin_dominant_score,
        pin_causal_row0_and_n1, pin_shift_and_permutation, pin_tiled_equals_direct,
        pin_torch_sdpa, pin_finite_differences, pin_autograd, pin_bwd_rows, pin_gradient_invariants,
        pin_large_spread]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(ref_module)


# ----------------------------------------------------------------------------
# planted mistakes: each broken copy of the oracle must fail at least one pin
# ----------------------------------------------------------------------------

def _mut_scores_no_scale(q, k, scale, causal):
    return _ORIG_SCORES(q, k, 1.0, causal)


def _mut_scores_transposed(q, k, scale, causal):
    s = _ORIG_SCORES(q, k, scale, False).T
    if causal:
        s = np.where(np.triu(np.ones(s.shape, dtype=bool), 1), -np.inf, s)
    return s


def _mut_scores_mask_leaks_one(q, k, scale, causal):
    s = scale * (q @ k.T)
    if causal:
        s = np.where(np.triu(np.ones(s.shape, dtype=bool), 2), -np.inf, s)
    return s


def _mut_scores_mask_wrong_side(q, k, scale, causal):
    s = scale * (q @ k.T)
    if causal:
        s = np.where(np.tril(np.ones(s.shape, dtype=bool), -1), -np.inf, s)
    return s


def _mut_softmax_no_max(s):
    f = np.exp(s)
    l = f.sum(axis=1, keepdims=True)
    return f / l, np.zeros(s.shape[0]), l[:, 0]


def _mut_softmax_lse_drops_max(s):
    p, m, l = _ORIG_SOFTMAX(s)
    return p, np.zeros_like(m), l


def _bwd_variant(kind):
    def bwd(q, k, v, do, scale, causal):
        q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        for b in range(q.shape[0]):
            for h in range(q.shape[1]):
                p = _ORIG_SOFTMAX(_ORIG_SCORES(q[b, h], k[b, h], scale, causal))[0]
                dv[b, h] = (p @ do[b, h]) if kind == "dv_untransposed" else p.T @ do[b, h]
                dp = do[b, h] @ v[b, h].T
                D = 0.0 if kind == "no_delta" else (p * dp).sum(axis=1, keepdims=True)
                ds = p * (dp - D) if kind != "delta_sign" else p * (dp + D)
                sq = 1.0 if kind == "dq_no_scale" else scale
                dq[b, h] = sq * (ds @ k[b, h])
                dk[b, h] = scale * ((ds @ q[b, h]) if kind == "dk_untransposed" else ds.T @ q[b, h])
        return dq, dk, dv
    return bwd


_ORIG_SCORES = ref_module._scores
_ORIG_SOFTMAX = ref_module._softmax_rows

MUTANTS = {
    "scores_no_scale": ("_scores", _mut_scores_no_scale),
    "scores_transposed": ("_scores", _mut_scores_transposed),
    "causal_mask_leaks_one_key": ("_scores", _mut_scores_mask_leaks_one),
    "causal_mask_wrong_side": ("_scores", _mut_scores_mask_wrong_side),
    "softmax_without_max": ("_softmax_rows", _mut_softmax_no_max),
    "lse_drops_max": ("_softmax_rows", _mut_softmax_lse_drops_max),
    "bwd_no_delta": ("ref_bwd", _bwd_variant("no_delta")),
    "bwd_delta_sign": ("ref_bwd", _bwd_variant("delta_sign")),
    "bwd_dq_no_scale": ("ref_bwd", _bwd_variant("dq_no_scale")),
    "bwd_dk_untransposed": ("ref_bwd", _bwd_variant("dk_untransposed")),
    "bwd_dv_untransposed": ("ref_bwd", _bwd_variant("dv_untransposed")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ref_module, attr, fn)
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(ref_module)
            except (AssertionError, FloatingPointError, ValueError):
                caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
