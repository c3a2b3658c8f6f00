"""fp64 CPU oracle for exact scaled-dot-product attention (forward and backward).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
helper or constant with the HIP library.

What it computes, and where the pages define it
-----------------------------------------------
The method is exact: the tiled, online-softmax kernel reaches the plain
attention result, only faster (FlashAttention-2 principle and deployment page
(yunthe.com), note after the tiled code; Journal of Software 2026(1) p.218
LLM pre-training survey, text around Eq. (1)-(2)).  So this oracle is the plain
definition written out, one (batch, head) at a time, with the N x N score and
probability matrices materialised in float64:

* scores ``S = scale * Q K^T``: FlashAttention optimisation page
  (intelliparadigm.com) section 1, steps 1-2 (scaling by 1/sqrt(d_k)); the
  scale is an argument so that any value can be checked.
* causal mask: key j is visible to query i iff j <= i (queries and keys have
  the same length, so top-left and bottom-right alignment coincide).  The
  pages only name the flag (``is_causal``, FlashAttention-2 page,
  troubleshooting item 3) and "masking" inside the fused block (Journal of
  Software survey, text after Eq. (2)).
* safe softmax (subtract the row maximum): FlashAttention-from-GPU-memory page
  (jsqmd.com) section 2.1; Journal of Software survey Eq. (1).
* ``O = P V``: FlashAttention optimisation page section 1, step 4.
* per-row log-sum-exp ``LSE_i = m_i + ln sum_j exp(S_ij - m_i)``: the
  normalisation statistics kept for the backward pass (FlashAttention
  optimisation page section 4.1; Journal of Software survey, the (m, l)
  statistics after Eq. (2)).  Natural logarithm, one value per query row.
* backward: the pages give only "recompute P from the saved statistics"
  (FlashAttention-from-GPU-memory page section 2.2; FlashAttention
  optimisation page section 4.2).  The gradients here are the chain rule on
  ``O = softmax(scale*QK^T + mask) V`` written out directly:
  ``dV = P^T dO``, ``dP = dO V^T``, ``D_i = sum_j P_ij dP_ij``,
  ``dS = P * (dP - D)``, ``dQ = scale * dS K``, ``dK = scale * dS^T Q``.

Every array argument is ``[B][H][N][d]`` (numpy, any float dtype; it is
widened to float64).  Results are float64.
"""
from __future__ import annotations

import numpy as np


def _scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool) -> np.ndarray:
    """Masked, scaled score matrix of one head: ``scale * q @ k.T``; masked -> -inf."""
    s = scale * (q @ k.T)
    if causal:
        n = s.shape[0]
        # key index > query index is hidden
        hidden = np.triu(np.ones((n, n), dtype=bool), k=1)
        s = np.where(hidden, -np.inf, s)
    return s


def _softmax_rows(s: np.ndarray):
    """Safe softmax of each row (subtract the row max, exponentiate, divide by the row sum).

    Returns ``(P, m, l)`` where ``m`` is the row max and ``l`` the row sum of
    ``exp(s - m)``; every row is assumed to hold at least one finite entry.
    """
    m = s.max(axis=1, keepdims=True)
    f = np.exp(s - m)  # exp(-inf) == 0 for hidden entries
    l = f.sum(axis=1, keepdims=True)
    return f / l, m[:, 0], l[:, 0]


def _as_f64(*arrays):
    return [np.asarray(a, dtype=np.float64) for a in arrays]


def ref_fwd(q, k, v, scale: float, causal: bool):
    """Forward attention: returns ``(O [B,H,N,d], LSE [B,H,N])`` in float64."""
    q, k, v = _as_f64(q, k, v)
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = _scores(q[b, h], k[b, h], scale, causal)
            p, m, l = _softmax_rows(s)
            o[b, h] = p @ v[b, h]
            lse[b, h] = m + np.log(l)
    return o, lse


def ref_fwd_rows(q, k, v, scale: float, causal: bool, rows):
    """Forward attention of one head ``[N,d]`` for the query rows ``rows`` only.

    Query rows are independent in the definition, so this is the same
    computation as ``ref_fwd`` restricted to a subset of rows (used to check
    outputs of workloads too large to materialise in full).  Returns
    ``(O[rows], LSE[rows])`` in float64.
    """
    q, k, v = _as_f64(q, k, v)
    rows = np.asarray(rows, dtype=np.int64)
    s = scale * (q[rows] @ k.T)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > rows[:, None], -np.inf, s)
    p, m, l = _softmax_rows(s)
    return p @ v, m + np.log(l)


def ref_probs(q, k, scale: float, causal: bool):
    """The attention probabilities ``P`` of every head, ``[B,H,N,N]`` (small inputs only)."""
    q, k = _as_f64(q, k)
    B, H, N, _ = q.shape
    out = np.empty((B, H, N, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = _softmax_rows(_scores(q[b, h], k[b, h], scale, causal))[0]
    return out


def ref_bwd(q, k, v, do, scale: float, causal: bool):
    """Backward attention: gradients of ``sum(O * dO)``; returns ``(dQ, dK, dV)`` in float64.

    P is recomputed from the inputs (the oracle keeps nothing between calls),
    masked entries have P = 0 and therefore contribute nothing.
    """
    q, k, v, do = _as_f64(q, k, v, do)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    B, H, _, _ = q.shape
    for b in range(B):
        for h in range(H):
            p = _softmax_rows(_scores(q[b, h], k[b, h], scale, causal))[0]
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            D = (p * dp).sum(axis=1, keepdims=True)
            ds = p * (dp - D)
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv


def ref_bwd_rows(q, k, v, do, scale: float, causal: bool, rows, keys):
    """One head ``[N,d]``: dQ of the query rows ``rows``, and what those rows add to dK and dV at the keys ``keys``.

    Every gradient term of a query row depends on that row alone (its P row,
    its dP row and its D_i), so ``dQ[rows]`` is ``ref_bwd``'s dQ restricted to
    the rows, and dK, dV are sums over the rows of per-row terms.  When the
    rows include every row that sees a key, the sums at that key are complete:
    the last T keys of a causal head are seen by the last T rows only.  Used on
    workloads too large to materialise in full.  Returns float64
    ``(dQ[rows], dK part [len(keys), d], dV part [len(keys), d])``.
    """
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    qr, dor = _as_f64(np.asarray(q)[rows], np.asarray(do)[rows])
    k, v = _as_f64(k, v)
    s = scale * (qr @ k.T)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > rows[:, None], -np.inf, s)
    p = _softmax_rows(s)[0]
    dp = dor @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return scale * (ds @ k), scale * (ds[:, keys].T @ qr), p[:, keys].T @ dor


def ref_bwd_delta(o, do):
    """``D_i = sum_k dO_ik * O_ik`` per row, ``[B,H,N]`` (equals ``sum_j P_ij dP_ij``)."""
    o, do = _as_f64(o, do)
    return (o * do).sum(axis=-1)
