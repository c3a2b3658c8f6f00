"""Pins of the window / block-sparse oracle (``oracle/masks.py``) against facts outside it.

* limits that reduce to the dense and causal definitions (``oracle.ref.ref_fwd``,
  pinned on its own): window (-1,-1) and (-1,0), an all-ones block mask with and
  without the causal flag;
* a block-diagonal mask equals independent attention inside each 64-row block
  (the dense definition applied to each block's slice of Q, K, V);
* per-row brute force over the visible keys of a window;
* constant keys: O is the mean of the visible V rows, LSE = scale q.k + ln(#visible);
* rows that see no key give O = 0 and LSE = -inf; per-head masks act per head.

Planted mistakes must each fail a pin.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle.masks as masks_module
import oracle.ref as ref_module


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).normal(0.0, std, size=shape)


def pin_window_limits(M):
    q, k, v = _rand((1, 2, 37, 8), 200, 1.5), _rand((1, 2, 37, 8), 201, 1.5), _rand((1, 2, 37, 8), 202)
    for (left, right), causal in (((-1, -1), False), ((-1, 0), True), ((36, 36), False), ((100, 0), True)):
        o, lse = M.ref_fwd_window(q, k, v, 0.3, left, right)
        ro, rl = ref_module.ref_fwd(q, k, v, 0.3, causal)
        np.testing.assert_allclose(o, ro, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-13)


def pin_window_brute_force(M):
    N, d = 11, 3
    q, k, v = _rand((1, 1, N, d), 210), _rand((1, 1, N, d), 211), _rand((1, 1, N, d), 212)
    for left, right in ((2, 3), (0, 0), (4, 0), (0, 5), (-1, 1), (3, -1)):
        o, lse = M.ref_fwd_window(q, k, v, 0.9, left, right)
        for i in range(N):
            vis = [j for j in range(N) if (left < 0 or j >= i - left) and (right < 0 or j <= i + right)]
            sc = [0.9 * sum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d)) for j in vis]
            mx = max(sc)
            ex = [math.exp(x - mx) for x in sc]
            tot = sum(ex)
            want = [sum(ex[n] * v[0, 0, j, t] for n, j in enumerate(vis)) / tot for t in range(d)]
            np.testing.assert_allclose(o[0, 0, i], want, rtol=0, atol=1e-14)
            assert abs(lse[0, 0, i] - (mx + math.log(tot))) < 1e-14


def pin_window_constant_keys(M):
    N, d = 29, 4
    q, v = _rand((1, 1, N, d), 220), _rand((1, 1, N, d), 221)
    kv = _rand((1, 1, 1, d), 222)
    k = np.repeat(kv, N, axis=2)
    left, right = 5, 2
    o, lse = M.ref_fwd_window(q, k, v, 0.5, left, right)
    for i in range(N):
        lo, hi = max(0, i - left), min(N - 1, i + right)
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, lo:hi + 1].mean(0), rtol=0, atol=1e-13)
        assert abs(lse[0, 0, i] - (0.5 * float(q[0, 0, i] @ kv[0, 0, 0]) + math.log(hi - lo + 1))) < 1e-13


def pin_blocksparse_limits(M):
    N = 150  # three 64-row blocks, the last one ragged
    q, k, v = _rand((1, 2, N, 8), 230, 1.5), _rand((1, 2, N, 8), 231, 1.5), _rand((1, 2, N, 8), 232)
    nb = 3
    for causal in (False, True):
        o, lse = M.ref_fwd_blocksparse(q, k, v, 0.3, causal, np.ones((nb, nb), np.uint8))
        ro, rl = ref_module.ref_fwd(q, k, v, 0.3, causal)
        np.testing.assert_allclose(o, ro, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-13)
    # block diagonal: each 64-row block attends to itself only
    o, lse = M.ref_fwd_blocksparse(q, k, v, 0.3, False, np.eye(nb, dtype=np.uint8))
    for b0 in range(0, N, 64):
        sl = slice(b0, min(N, b0 + 64))
        ro, rl = ref_module.ref_fwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.3, False)
        np.testing.assert_allclose(o[:, :, sl], ro, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, sl], rl, rtol=0, atol=1e-13)
    # keys of block 1 only, for every query block: attention over that slice of keys
    bm = np.zeros((nb, nb), np.uint8)
    bm[:, 1] = 1
    o, lse = M.ref_fwd_blocksparse(q, k, v, 0.3, False, bm)
    s = 0.3 * np.einsum("bhid,bhjd->bhij", q, k[:, :, 64:128])
    mx = s.max(-1, keepdims=True)
    p = np.exp(s - mx)
    np.testing.assert_allclose(o, (p @ v[:, :, 64:128]) / p.sum(-1, keepdims=True), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, mx[..., 0] + np.log(p.sum(-1)), rtol=0, atol=1e-13)


def pin_blocksparse_empty_rows_and_heads(M):
    N = 128
    q, k, v = _rand((1, 2, N, 4), 240), _rand((1, 2, N, 4), 241), _rand((1, 2, N, 4), 242)
    bm = np.array([[[1, 1], [0, 0]], [[0, 0], [1, 0]]], np.uint8)  # head 0: block row 1 empty; head 1: row 0
    o, lse = M.ref_fwd_blocksparse(q, k, v, 0.4, False, bm)
    assert np.all(o[0, 0, 64:] == 0) and np.all(lse[0, 0, 64:] == -np.inf)
    assert np.all(o[0, 1, :64] == 0) and np.all(lse[0, 1, :64] == -np.inf)
    ro, rl = ref_module.ref_fwd(q[:, :1, :64], k[:, :1], v[:, :1], 0.4, False)
    np.testing.assert_allclose(o[:, :1, :64], ro, rtol=0, atol=1e-13)
    s = 0.4 * np.einsum("id,jd->ij", q[0, 1, 64:], k[0, 1, :64])
    mx = s.max(-1, keepdims=True)
    p = np.exp(s - mx)
    np.testing.assert_allclose(o[0, 1, 64:], (p @ v[0, 1, :64]) / p.sum(-1, keepdims=True), rtol=0, atol=1e-13)
    # causal on top of a block that lies above the diagonal leaves row 0 of head 0 only its own key
    o2, lse2 = M.ref_fwd_blocksparse(q, k, v, 0.4, True, bm)
    np.testing.assert_allclose(o2[0, 0, 0], v[0, 0, 0], rtol=0, atol=1e-15)
    assert np.all(lse2[0, 1, :64] == -np.inf)


def pin_row_variants_match(M):
    """The row-subset versions (used on workloads too large for full N x N) agree
    with the full ones, themselves pinned above."""
    N = 200
    q, k, v = _rand((1, 1, N, 6), 250, 1.5), _rand((1, 1, N, 6), 251, 1.5), _rand((1, 1, N, 6), 252)
    rows = np.array([0, 1, 63, 64, 65, 127, 150, 199])
    for left, right in ((10, 3), (-1, 0), (0, -1)):
        o, lse = M.ref_fwd_window(q, k, v, 0.4, left, right)
        orow, lrow = M.ref_fwd_window_rows(q[0, 0], k[0, 0], v[0, 0], 0.4, left, right, rows)
        np.testing.assert_allclose(orow, o[0, 0, rows], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lrow, lse[0, 0, rows], rtol=0, atol=1e-14)
    bm = (np.random.default_rng(253).random((4, 4)) < 0.5).astype(np.uint8)
    bm[1] = 0
    for causal in (False, True):
        o, lse = M.ref_fwd_blocksparse(q, k, v, 0.4, causal, bm)
        orow, lrow = M.ref_fwd_blocksparse_rows(q[0, 0], k[0, 0], v[0, 0], 0.4, causal, bm, rows)
        np.testing.assert_allclose(orow, o[0, 0, rows], rtol=0, atol=1e-14)
        np.testing.assert_array_equal(np.isinf(lrow), np.isinf(lse[0, 0, rows]))
        fin = np.isfinite(lrow)
        np.testing.assert_allclose(lrow[fin], lse[0, 0, rows][fin], rtol=0, atol=1e-14)


PINS = [pin_window_limits, pin_window_brute_force, pin_window_constant_keys, pin_blocksparse_limits,
        pin_blocksparse_empty_rows_and_heads, pin_row_variants_match]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_mask_oracle_pin(pin):
    pin(masks_module)


_ORIG_WIN = masks_module.window_visible
_ORIG_BLK = masks_module.blocksparse_visible


def _mut_window_off_by_one(N, left, right):
    return _ORIG_WIN(N, left + 1 if left >= 0 else left, right)


def _mut_window_sides_swapped(N, left, right):
    return _ORIG_WIN(N, right, left)


def _mut_block_transposed(N, block_mask, causal):
    return _ORIG_BLK(N, np.asarray(block_mask).T, causal)


def _mut_block_ignores_causal(N, block_mask, causal):
    return _ORIG_BLK(N, block_mask, False)


def _mut_block_size_32(N, block_mask, causal):
    bm = np.asarray(block_mask) != 0
    qb = np.minimum(np.arange(N) // 32, bm.shape[0] - 1)
    vis = bm[qb[:, None], qb[None, :]]
    if causal:
        vis &= np.arange(N)[None, :] <= np.arange(N)[:, None]
    return vis


MUTANTS = {
    "window_off_by_one": ("window_visible", _mut_window_off_by_one),
    "window_sides_swapped": ("window_visible", _mut_window_sides_swapped),
    "block_mask_transposed": ("blocksparse_visible", _mut_block_transposed),
    "block_ignores_causal": ("blocksparse_visible", _mut_block_ignores_causal),
    "block_size_32": ("blocksparse_visible", _mut_block_size_32),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mask_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(masks_module, attr, fn)
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(masks_module)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
