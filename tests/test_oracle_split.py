"""Pins of the split-key oracle (``oracle/split.py``) against facts outside it.

* merging the parts of any cut of the keys reproduces the direct attention
  result (``oracle.ref.ref_fwd``, pinned on its own in ``test_oracle.py``): the
  claim of Eq. (2) of the Journal of Software survey;
* the key-range forward equals per-row brute force over the visible keys, and
  a closed form for constant keys;
* closed forms of the merge: one part is returned unchanged, two equal parts
  give the same O and LSE + ln 2, parts with LSE = -inf are ignored;
* the pairwise (m, l) statistics of Eq. (2) (``oracle.online_softmax``) fold to
  the same LSE as the S-way merge.

Planted mistakes in broken copies of the two functions must each fail a pin.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle.ref as ref_module
import oracle.split as split_module
from oracle import online_softmax as osm


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).normal(0.0, std, size=shape)


CUTS = {
    23: [[0, 23], [0, 7, 23], [0, 1, 9, 16, 23], [0, 11, 12, 23], [0, 5, 10, 15, 20, 23]],
    64: [[0, 64], [0, 32, 64], [0, 13, 40, 64]],
}


def _parts(S, q, k, v, scale, causal, cut):
    outs = [S.ref_fwd_keyrange(q, k, v, scale, causal, a, b) for a, b in zip(cut[:-1], cut[1:])]
    return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])


def pin_merge_of_parts_equals_direct(S):
    for N, cuts in CUTS.items():
        q, k, v = _rand((1, 2, N, 8), 100 + N, 1.5), _rand((1, 2, N, 8), 101 + N, 1.5), _rand((1, 2, N, 8), 102 + N)
        for causal in (False, True):
            o, lse = ref_module.ref_fwd(q, k, v, 0.4, causal)
            for cut in cuts:
                op, lp = _parts(S, q, k, v, 0.4, causal, cut)
                om, lm = S.ref_lse_merge(op, lp)
                np.testing.assert_allclose(om, o, rtol=0, atol=1e-13)
                np.testing.assert_allclose(lm, lse, rtol=0, atol=1e-13)


def pin_keyrange_brute_force(S):
    N, d = 9, 3
    q, k, v = _rand((1, 1, N, d), 110), _rand((1, 1, N, d), 111), _rand((1, 1, N, d), 112)
    for causal in (False, True):
        for k0, k1 in ((0, N), (2, 5), (4, 9), (3, 4), (6, 6)):
            o, lse = S.ref_fwd_keyrange(q, k, v, 0.8, causal, k0, k1)
            for i in range(N):
                vis = [j for j in range(k0, k1) if not causal or j <= i]
                if not vis:
                    assert lse[0, 0, i] == -math.inf and np.all(o[0, 0, i] == 0)
                    continue
                sc = [0.8 * sum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d)) for j in vis]
                mx = max(sc)
                ex = [math.exp(x - mx) for x in sc]
                tot = sum(ex)
                want = [sum(ex[n] * v[0, 0, j, t] for n, j in enumerate(vis)) / tot for t in range(d)]
                np.testing.assert_allclose(o[0, 0, i], want, rtol=0, atol=1e-14)
                assert abs(lse[0, 0, i] - (mx + math.log(tot))) < 1e-14


def pin_keyrange_constant_keys(S):
    N, d = 17, 5
    q, v = _rand((1, 1, N, d), 120), _rand((1, 1, N, d), 121)
    kv = _rand((1, 1, 1, d), 122)
    k = np.repeat(kv, N, axis=2)
    for causal in (False, True):
        o, lse = S.ref_fwd_keyrange(q, k, v, 0.5, causal, 4, 13)
        for i in range(N):
            hi = min(13, i + 1) if causal else 13
            n = hi - 4
            if n <= 0:
                assert lse[0, 0, i] == -math.inf
                continue
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, 4:hi].mean(0), rtol=0, atol=1e-13)
            assert abs(lse[0, 0, i] - (0.5 * float(q[0, 0, i] @ kv[0, 0, 0]) + math.log(n))) < 1e-13


def pin_merge_closed_forms(S):
    o1, l1 = _rand((1, 2, 6, 4), 130), _rand((1, 2, 6), 131, 3.0)
    om, lm = S.ref_lse_merge(o1[None], l1[None])
    np.testing.assert_allclose(om, o1, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lm, l1, rtol=0, atol=1e-15)
    om, lm = S.ref_lse_merge(np.stack([o1, o1]), np.stack([l1, l1]))
    np.testing.assert_allclose(om, o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lm, l1 + math.log(2), rtol=0, atol=1e-14)
    # two parts with LSE a and b: weights e^a/(e^a+e^b) and e^b/(e^a+e^b)
    o2, l2 = _rand((1, 2, 6, 4), 132), _rand((1, 2, 6), 133, 3.0)
    om, lm = S.ref_lse_merge(np.stack([o1, o2]), np.stack([l1, l2]))
    w1 = 1.0 / (1.0 + np.exp(l2 - l1))
    np.testing.assert_allclose(om, w1[..., None] * o1 + (1 - w1[..., None]) * o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lm, np.logaddexp(l1, l2), rtol=0, atol=1e-13)
    # a part that saw no key is ignored, whatever its O holds
    empty_l = np.full_like(l1, -np.inf)
    om, lm = S.ref_lse_merge(np.stack([o1, np.full_like(o1, 7.0), o2]), np.stack([l1, empty_l, l2]))
    np.testing.assert_allclose(om, w1[..., None] * o1 + (1 - w1[..., None]) * o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lm, np.logaddexp(l1, l2), rtol=0, atol=1e-13)
    # large LSE values must not overflow
    om, lm = S.ref_lse_merge(np.stack([o1, o2]), np.stack([l1 + 800.0, l2 + 800.0]))
    assert np.all(np.isfinite(om)) and np.all(np.isfinite(lm))
    np.testing.assert_allclose(lm, np.logaddexp(l1, l2) + 800.0, rtol=0, atol=1e-12)


def pin_pairwise_eq2_matches_merge(S):
    x = _rand(40, 140, 2.0)
    cuts = [0, 6, 17, 18, 40]
    blocks = [x[a:b] for a, b in zip(cuts[:-1], cuts[1:])]
    stats = None
    for bk in blocks:
        st = osm.block_stats(bk)
        stats = st if stats is None else osm.merge_stats(stats, st)
    m, _, l = stats
    lse_parts = np.array([float(np.log(np.sum(np.exp(bk - bk.max())))) + float(bk.max()) for bk in blocks])
    dummy = np.zeros((len(blocks), 1, 1, 1, 1))
    _, lm = S.ref_lse_merge(dummy, lse_parts.reshape(-1, 1, 1, 1))
    assert abs(float(lm[0, 0, 0]) - (m + math.log(l))) < 1e-13


PINS = [pin_merge_of_parts_equals_direct, pin_keyrange_brute_force, pin_keyrange_constant_keys,
        pin_merge_closed_forms, pin_pairwise_eq2_matches_merge]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_split_oracle_pin(pin):
    pin(split_module)


# ----------------------------------------------------------------------------
# planted mistakes
# ----------------------------------------------------------------------------

_ORIG_MERGE = split_module.ref_lse_merge
_ORIG_RANGE = split_module.ref_fwd_keyrange


def _mut_merge_unnormalised(o_parts, lse_parts):
    o, lse = _ORIG_MERGE(o_parts, lse_parts)
    return o * np.exp(lse - np.max(lse_parts, axis=0))[..., None], lse


def _mut_merge_plain_mean(o_parts, lse_parts):
    o, lse = _ORIG_MERGE(o_parts, lse_parts)
    return np.mean(o_parts, axis=0), lse


def _mut_merge_lse_drops_max(o_parts, lse_parts):
    o, lse = _ORIG_MERGE(o_parts, lse_parts)
    return o, lse - np.max(lse_parts, axis=0)


def _mut_merge_weights_swapped(o_parts, lse_parts):
    return _ORIG_MERGE(o_parts, -lse_parts)[0], _ORIG_MERGE(o_parts, lse_parts)[1]


def _mut_range_inclusive_end(q, k, v, scale, causal, k0, k1):
    return _ORIG_RANGE(q, k, v, scale, causal, k0, k1 + 1)


def _mut_range_ignores_causal(q, k, v, scale, causal, k0, k1):
    return _ORIG_RANGE(q, k, v, scale, False, k0, k1)


MUTANTS = {
    "merge_unnormalised": ("ref_lse_merge", _mut_merge_unnormalised),
    "merge_plain_mean": ("ref_lse_merge", _mut_merge_plain_mean),
    "merge_lse_drops_max": ("ref_lse_merge", _mut_merge_lse_drops_max),
    "merge_weights_swapped": ("ref_lse_merge", _mut_merge_weights_swapped),
    "range_inclusive_end": ("ref_fwd_keyrange", _mut_range_inclusive_end),
    "range_ignores_causal": ("ref_fwd_keyrange", _mut_range_ignores_causal),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_split_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(split_module, attr, fn)
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(split_module)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
