"""Pins of the masked backward oracle (``oracle/masks.py``: ``ref_bwd_window``,
``ref_bwd_blocksparse``) against facts outside its own arithmetic.

* limits: window (-1,-1) / (-1,0) and an all-ones block mask (with and without
  the causal flag) reduce to the dense and causal gradients of
  ``oracle.ref.ref_bwd`` (pinned on its own);
* finite differences of ``sum(O * dO)`` through the masked forward (pinned on
  its own), for windows and for a block mask with causal on top and with a
  query block that sees no key;
* a block-diagonal mask equals independent dense gradients inside each block;
* rows that see no key: their dQ rows are exactly 0 and their dO does not
  reach dK or dV;
* invariants that hold under any mask: every row of dS sums to 0, so the dK
  rows sum to 0; the dV rows sum to the dO rows of the rows that see a key.

Planted mistakes in the chain rule and in the visibility must each fail a pin.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle.masks as M
import oracle.ref as ref_module


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).normal(0.0, std, size=shape)


def _inputs(B, H, N, d, seed, std=1.0):
    return tuple(_rand((B, H, N, d), seed + i, std if i < 2 else 1.0) for i in range(4))


def pin_bwd_limits(m):
    q, k, v, do = _inputs(1, 2, 37, 8, 300, 1.5)
    for (left, right), causal in (((-1, -1), False), ((-1, 0), True), ((36, 36), False), ((100, 0), True)):
        got = m.ref_bwd_window(q, k, v, do, 0.3, left, right)
        want = ref_module.ref_bwd(q, k, v, do, 0.3, causal)
        for g, w in zip(got, want):
            np.testing.assert_allclose(g, w, rtol=0, atol=1e-12)
    q, k, v, do = _inputs(1, 2, 150, 8, 310, 1.5)
    for causal in (False, True):
        got = m.ref_bwd_blocksparse(q, k, v, do, 0.3, causal, np.ones((3, 3), np.uint8))
        want = ref_module.ref_bwd(q, k, v, do, 0.3, causal)
        for g, w in zip(got, want):
            np.testing.assert_allclose(g, w, rtol=0, atol=1e-12)


def _fd_check(loss, grads, tensors, rng, count=6, eps=1e-6, tol=2e-7):
    for t, g in zip(tensors, grads):
        flat = t.reshape(-1)
        for idx in rng.choice(flat.size, size=min(count, flat.size), replace=False):
            old = flat[idx]
            flat[idx] = old + eps
            up = loss()
            flat[idx] = old - eps
            dn = loss()
            flat[idx] = old
            fd = (up - dn) / (2 * eps)
            assert abs(fd - g.reshape(-1)[idx]) <= tol * max(1.0, abs(fd)), (idx, fd, g.reshape(-1)[idx])


def pin_bwd_finite_differences(m):
    rng = np.random.default_rng(320)
    q, k, v, do = _inputs(1, 1, 9, 3, 321)
    for left, right in ((2, 1), (0, 3), (-1, 2), (1, -1)):
        grads = m.ref_bwd_window(q, k, v, do, 0.7, left, right)
        loss = lambda: float((m.ref_fwd_window(q, k, v, 0.7, left, right)[0] * do).sum())  # noqa: E731
        _fd_check(loss, grads, (q, k, v), rng)
    q, k, v, do = _inputs(1, 2, 130, 2, 330)
    bm = np.array([[[1, 0, 1], [0, 0, 0], [1, 1, 0]], [[0, 1, 0], [1, 1, 0], [0, 1, 1]]], np.uint8)
    for causal in (False, True):
        grads = m.ref_bwd_blocksparse(q, k, v, do, 0.5, causal, bm)
        loss = lambda: float((np.nan_to_num(m.ref_fwd_blocksparse(q, k, v, 0.5, causal, bm)[0]) * do).sum())  # noqa: E731
        _fd_check(loss, grads, (q, k, v), rng, count=8)


def pin_bwd_block_diagonal(m):
    N = 150
    q, k, v, do = _inputs(1, 2, N, 6, 340, 1.5)
    got = m.ref_bwd_blocksparse(q, k, v, do, 0.4, False, np.eye(3, dtype=np.uint8))
    for b0 in range(0, N, 64):
        sl = slice(b0, min(N, b0 + 64))
        want = ref_module.ref_bwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], do[:, :, sl], 0.4, False)
        for g, w in zip(got, want):
            np.testing.assert_allclose(g[:, :, sl], w, rtol=0, atol=1e-12)


def pin_bwd_empty_rows(m):
    N = 128
    q, k, v, do = _inputs(1, 2, N, 4, 350)
    bm = np.array([[[1, 1], [0, 0]], [[0, 0], [1, 0]]], np.uint8)  # head 0: rows 64.. empty; head 1: rows 0..63
    dq, dk, dv = m.ref_bwd_blocksparse(q, k, v, do, 0.4, False, bm)
    assert np.all(dq[0, 0, 64:] == 0) and np.all(dq[0, 1, :64] == 0)
    do2 = do.copy()
    do2[0, 0, 64:] = _rand((N - 64, 4), 351)
    do2[0, 1, :64] = 0.0
    _, dk2, dv2 = m.ref_bwd_blocksparse(q, k, v, do2, 0.4, False, bm)
    np.testing.assert_allclose(dk2, dk, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv2, dv, rtol=0, atol=1e-13)


def pin_bwd_sum_invariants(m):
    N = 200
    q, k, v, do = _inputs(1, 2, N, 5, 360, 2.0)
    nb = 4
    bm = (np.random.default_rng(361).random((2, nb, nb)) < 0.5).astype(np.uint8)
    bm[0, 2] = 0
    cases = [(m.ref_bwd_window(q, k, v, do, 0.6, 7, 3), M.window_visible(N, 7, 3)),
             (m.ref_bwd_blocksparse(q, k, v, do, 0.6, True, bm),
              np.stack([M.blocksparse_visible(N, bm[h], True) for h in range(2)]))]
    for (dq, dk, dv), vis in cases:
        for h in range(2):
            vish = vis if vis.ndim == 2 else vis[h]
            seen = vish.any(axis=1)
            np.testing.assert_allclose(dk[0, h].sum(0), 0.0, rtol=0, atol=1e-11)
            np.testing.assert_allclose(dv[0, h].sum(0), do[0, h][seen].sum(0), rtol=0, atol=1e-11)


PINS = [pin_bwd_limits, pin_bwd_finite_differences, pin_bwd_block_diagonal, pin_bwd_empty_rows,
        pin_bwd_sum_invariants]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_masked_bwd_oracle_pin(pin):
    pin(M)


_ORIG_GRADS = M._grads_from_probs
_ORIG_PROBS = M._visible_probs
_ORIG_WIN = M.window_visible
_ORIG_BLK = M.blocksparse_visible


def _mut_no_delta(p, q, k, v, do, scale):
    dv = p.T @ do
    ds = p * (do @ v.T)
    return scale * (ds @ k), scale * (ds.T @ q), dv


def _mut_dk_untransposed(p, q, k, v, do, scale):
    dq, _, dv = _ORIG_GRADS(p, q, k, v, do, scale)
    dv_ = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return dq, scale * (ds @ q), dv_


def _mut_dv_untransposed(p, q, k, v, do, scale):
    dq, dk, _ = _ORIG_GRADS(p, q, k, v, do, scale)
    return dq, dk, p @ do


def _mut_dq_unscaled(p, q, k, v, do, scale):
    dq, dk, dv = _ORIG_GRADS(p, q, k, v, do, scale)
    return dq / scale, dk, dv


def _mut_probs_unmasked(q, k, scale, vis):
    return _ORIG_PROBS(q, k, scale, np.ones_like(vis))


def _mut_window_sides_swapped(N, left, right):
    return _ORIG_WIN(N, right, left)


def _mut_block_transposed(N, block_mask, causal):
    return _ORIG_BLK(N, np.asarray(block_mask).T, causal)


MUTANTS = {
    "no_delta_term": ("_grads_from_probs", _mut_no_delta),
    "dk_untransposed": ("_grads_from_probs", _mut_dk_untransposed),
    "dv_untransposed": ("_grads_from_probs", _mut_dv_untransposed),
    "dq_unscaled": ("_grads_from_probs", _mut_dq_unscaled),
    "probs_ignore_mask": ("_visible_probs", _mut_probs_unmasked),
    "window_sides_swapped": ("window_visible", _mut_window_sides_swapped),
    "block_mask_transposed": ("blocksparse_visible", _mut_block_transposed),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_masked_bwd_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(M, attr, fn)
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(M)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
