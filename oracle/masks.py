"""fp64 oracle for attention under sliding-window and block-sparse masks.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle/ref.py``).

The pages name two ways of skipping whole blocks of the score matrix: a
sliding window around each query (the FlashAttention-2 principle and
deployment page, section on SDPA usage, passes ``window_size=(512, 512)``) and
block-sparse FlashAttention (FlashAttention optimisation page, section 7;
Journal of Software survey, the sparse-attention sentence after Eq. (2)).
Neither page defines the mask precisely; the readings written out here are:

* sliding window ``(left, right)``: key j is visible to query i iff
  ``i - left <= j <= i + right``; a negative bound means no limit on that
  side, so ``(-1, -1)`` is dense attention and ``(-1, 0)`` is the causal mask.
  Every query sees at least itself.
* block-sparse: the N x N score matrix is cut into 64 x 64 blocks (query block
  ``i // 64``, key block ``j // 64``); ``block_mask[h][qb][kb] != 0`` keeps the
  block, 0 drops it.  With ``causal`` the usual ``j <= i`` applies on top.

Within the visible set the computation is the plain definition of
``oracle/ref.py``.  A row with no visible key (possible only with a block
mask) has an empty softmax; its output is taken as ``O = 0`` and its
log-sum-exp as ``-inf`` (the sum over an empty set is 0).

The backward under a mask is the chain rule on that forward, as for the dense
case (recompute P, then dV = P^T dO, dP = dO V^T, dS = P * (dP - D) with
D_i = sum_j P_ij dP_ij, dQ = scale dS K, dK = scale dS^T Q): hidden entries
have P = 0 and so add nothing, and a row with no visible key has a constant
output O = 0, so it contributes nothing to any gradient and its dQ row is 0.
"""
from __future__ import annotations

import numpy as np

from .ref import _as_f64

MASK_BLOCK = 64


def window_visible(N: int, left: int, right: int) -> np.ndarray:
    """``[N, N]`` bool: key j visible to query i iff i-left <= j <= i+right (negative = unlimited)."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    vis = np.ones((N, N), dtype=bool)
    if left >= 0:
        vis &= j >= i - left
    if right >= 0:
        vis &= j <= i + right
    return vis


def blocksparse_visible(N: int, block_mask: np.ndarray, causal: bool) -> np.ndarray:
    """``[N, N]`` bool from a ``[nb, nb]`` block mask of 64 x 64 blocks (plus j <= i if causal)."""
    bm = np.asarray(block_mask) != 0
    qb = np.arange(N) // MASK_BLOCK
    vis = bm[qb[:, None], qb[None, :]]
    if causal:
        vis &= np.arange(N)[None, :] <= np.arange(N)[:, None]
    return vis


def ref_fwd_visible(q, k, v, scale: float, visible):
    """Attention with an explicit visibility matrix ``[N,N]`` (all heads) or ``[H,N,N]``.

    Returns ``(O [B,H,N,d], LSE [B,H,N])`` in float64; rows with no visible
    key get ``O = 0`` and ``LSE = -inf``.
    """
    q, k, v = _as_f64(q, k, v)
    B, H, N, _ = q.shape
    visible = np.asarray(visible, dtype=bool)
    o = np.zeros((B, H, N, v.shape[-1]))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            vis = visible if visible.ndim == 2 else visible[h]
            s = np.where(vis, scale * (q[b, h] @ k[b, h].T), -np.inf)
            m = s.max(axis=1)
            seen = m > -np.inf
            if not seen.any():
                continue
            f = np.exp(s[seen] - m[seen, None])
            l = f.sum(axis=1)
            o[b, h, seen] = (f @ v[b, h]) / l[:, None]
            lse[b, h, seen] = m[seen] + np.log(l)
    return o, lse


def ref_fwd_window(q, k, v, scale: float, left: int, right: int):
    """Sliding-window attention; see the module notes for the reading of the window."""
    return ref_fwd_visible(q, k, v, scale, window_visible(np.shape(q)[2], left, right))


def ref_fwd_blocksparse(q, k, v, scale: float, causal: bool, block_mask):
    """Block-sparse attention; ``block_mask`` is ``[nb,nb]`` (every head) or ``[H,nb,nb]``."""
    N = np.shape(q)[2]
    bm = np.asarray(block_mask)
    if bm.ndim == 2:
        return ref_fwd_visible(q, k, v, scale, blocksparse_visible(N, bm, causal))
    return ref_fwd_visible(q, k, v, scale, np.stack([blocksparse_visible(N, m, causal) for m in bm]))


def _rows_fwd(q, k, v, scale: float, vis):
    """One head: attention of the query rows whose visibility rows are ``vis [R, N]``."""
    s = np.where(vis, scale * (q @ k.T), -np.inf)
    m = s.max(axis=1)
    o = np.zeros((s.shape[0], v.shape[-1]))
    lse = np.full(s.shape[0], -np.inf)
    seen = m > -np.inf
    if seen.any():
        f = np.exp(s[seen] - m[seen, None])
        l = f.sum(axis=1)
        o[seen] = (f @ v) / l[:, None]
        lse[seen] = m[seen] + np.log(l)
    return o, lse


def ref_fwd_window_rows(q, k, v, scale: float, left: int, right: int, rows):
    """Sliding-window attention of one head ``[N,d]`` for the query rows ``rows`` only."""
    q, k, v = _as_f64(q, k, v)
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(k.shape[0])[None, :]
    i = rows[:, None]
    vis = np.ones((rows.size, k.shape[0]), dtype=bool)
    if left >= 0:
        vis &= j >= i - left
    if right >= 0:
        vis &= j <= i + right
    return _rows_fwd(q[rows], k, v, scale, vis)


def ref_fwd_blocksparse_rows(q, k, v, scale: float, causal: bool, block_mask, rows):
    """Block-sparse attention of one head ``[N,d]`` (``block_mask [nb,nb]``) for ``rows`` only."""
    q, k, v = _as_f64(q, k, v)
    rows = np.asarray(rows, dtype=np.int64)
    bm = np.asarray(block_mask) != 0
    kb = np.arange(k.shape[0]) // MASK_BLOCK
    vis = bm[(rows // MASK_BLOCK)[:, None], kb[None, :]]
    if causal:
        vis &= np.arange(k.shape[0])[None, :] <= rows[:, None]
    return _rows_fwd(q[rows], k, v, scale, vis)


def _visible_probs(q, k, scale: float, vis):
    """One head: ``P [R, N]`` of the query rows whose visibility rows are ``vis``; empty rows are 0."""
    s = np.where(vis, scale * (q @ k.T), -np.inf)
    m = s.max(axis=1)
    p = np.zeros_like(s)
    seen = m > -np.inf
    if seen.any():
        f = np.exp(s[seen] - m[seen, None])
        p[seen] = f / f.sum(axis=1, keepdims=True)
    return p


def _grads_from_probs(p, q, k, v, do, scale: float):
    """Chain rule of one head from its probabilities: ``(dQ, dK, dV)``."""
    dv = p.T @ do
    dp = do @ v.T
    D = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - D)
    return scale * (ds @ k), scale * (ds.T @ q), dv


def ref_bwd_visible(q, k, v, do, scale: float, visible):
    """Gradients ``(dQ, dK, dV)`` of ``sum(O * dO)`` for ``ref_fwd_visible``'s attention, float64."""
    q, k, v, do = _as_f64(q, k, v, do)
    B, H, _, _ = q.shape
    visible = np.asarray(visible, dtype=bool)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(B):
        for h in range(H):
            vis = visible if visible.ndim == 2 else visible[h]
            p = _visible_probs(q[b, h], k[b, h], scale, vis)
            dq[b, h], dk[b, h], dv[b, h] = _grads_from_probs(p, q[b, h], k[b, h], v[b, h], do[b, h], scale)
    return dq, dk, dv


def ref_bwd_window(q, k, v, do, scale: float, left: int, right: int):
    """Gradients of sliding-window attention (the window read as in ``window_visible``)."""
    return ref_bwd_visible(q, k, v, do, scale, window_visible(np.shape(q)[2], left, right))


def ref_bwd_blocksparse(q, k, v, do, scale: float, causal: bool, block_mask):
    """Gradients of block-sparse attention; ``block_mask`` is ``[nb,nb]`` or ``[H,nb,nb]``."""
    N = np.shape(q)[2]
    bm = np.asarray(block_mask)
    if bm.ndim == 2:
        return ref_bwd_visible(q, k, v, do, scale, blocksparse_visible(N, bm, causal))
    return ref_bwd_visible(q, k, v, do, scale, np.stack([blocksparse_visible(N, m, causal) for m in bm]))
