"""Block-wise online softmax, written from its equations, for checking the direct oracle.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle/ref.py``: only tests, the smoke
check and the CPU-baseline leg of the benchmark may use it).

The method's central claim is that attention computed one key block at a time,
carrying a running maximum and a running sum, equals the direct softmax exactly
(up to rounding).  This module restates that computation in plain Python/NumPy
so that a test can compare it with ``oracle.ref.ref_fwd`` on tiny inputs:

* ``block_stats`` is Eq. (1) of the Journal of Software 2026(1) p.218 LLM
  pre-training survey: for one block x, ``m(x)`` is its maximum, ``f(x)`` the
  vector of ``exp(x_i - m(x))`` and ``l(x)`` the sum of ``f(x)``.
* ``merge_stats`` is Eq. (2) of the same page: two blocks with statistics
  ``(m1, f1, l1)`` and ``(m2, f2, l2)`` combine into ``m = max(m1, m2)``,
  ``f = [e^(m1-m) f1, e^(m2-m) f2]`` and ``l = e^(m1-m) l1 + e^(m2-m) l2``.
* ``tiled_attention_fwd`` applies the same merge to attention rows, with the
  partial output rescaled by the same factor as the partial sum (the tiled
  forward of the FlashAttention-2 principle and deployment page, first code
  section, and the forward steps of the FlashAttention optimisation page,
  section 4.1), and divides by the final sum at the end.  Blocks of queries
  and of keys may have any size, including sizes that do not divide N.
* ``two_pass_softmax`` is the variant of the FlashAttention-from-GPU-memory
  page (section 2.1) that finds the global maximum over all blocks first and
  then sums block by block.

A block whose scores are all masked (-inf) has ``m = -inf``; the merge then
uses a factor of 0 for it (e^(-inf) = 0), which is the limit of Eq. (2).
"""
from __future__ import annotations

import math

import numpy as np


def block_stats(x: np.ndarray):
    """Eq. (1): ``(m, f, l)`` of one block (1-D float64 array)."""
    m = float(np.max(x)) if x.size else -math.inf
    if m == -math.inf:
        f = np.zeros_like(x)
    else:
        f = np.exp(x - m)
    return m, f, float(np.sum(f))


def _factor(m_part: float, m_all: float) -> float:
    """``e^(m_part - m_all)``, taken as 0 for an all-masked part."""
    if m_part == -math.inf:
        return 0.0
    return math.exp(m_part - m_all)


def merge_stats(a, b):
    """Eq. (2): statistics of the concatenation of two blocks."""
    m1, f1, l1 = a
    m2, f2, l2 = b
    m = max(m1, m2)
    c1 = _factor(m1, m)
    c2 = _factor(m2, m)
    f = np.concatenate([c1 * f1, c2 * f2])
    return m, f, c1 * l1 + c2 * l2


def online_softmax(x: np.ndarray, block: int) -> np.ndarray:
    """Softmax of a 1-D vector by folding Eq. (2) over blocks of ``block`` entries."""
    stats = None
    for start in range(0, x.size, block):
        s = block_stats(x[start:start + block])
        stats = s if stats is None else merge_stats(stats, s)
    m, f, l = stats
    return f / l


def two_pass_softmax(x: np.ndarray, block: int) -> np.ndarray:
    """Global maximum over all blocks first, then per-block sums, then normalise."""
    blocks = [x[s:s + block] for s in range(0, x.size, block)]
    g = max(float(np.max(bk)) for bk in blocks)
    total = sum(float(np.sum(np.exp(bk - g))) for bk in blocks)
    return np.concatenate([np.exp(bk - g) / total for bk in blocks])


def tiled_attention_fwd(q, k, v, scale: float, causal: bool, block_q: int, block_k: int):
    """Attention of ``[B,H,N,d]`` inputs computed tile by tile with running (m, l, O).

    Loops: query blocks outside, key blocks inside; per key block the scores of
    the tile are formed, the running max is raised, the old partial sum and
    partial output are scaled by ``e^(m_old - m_new)`` and the tile's
    ``exp(S - m_new)`` terms are added.  The output is ``O / l`` and the
    statistic is ``m + ln l``.  Pure Python loops over rows: tiny inputs only.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, N, dv))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i0 in range(0, N, block_q):
                rows = range(i0, min(i0 + block_q, N))
                m = {r: -math.inf for r in rows}
                l = {r: 0.0 for r in rows}
                acc = {r: np.zeros(dv) for r in rows}
                for j0 in range(0, N, block_k):
                    cols = list(range(j0, min(j0 + block_k, N)))
                    for r in rows:
                        s = np.array([scale * float(q[b, h, r] @ k[b, h, c])
                                      if (not causal or c <= r) else -math.inf
                                      for c in cols])
                        m_new = max(m[r], float(np.max(s)))
                        if m_new == -math.inf:
                            continue  # nothing visible yet in this row
                        alpha = _factor(m[r], m_new)
                        p = np.exp(s - m_new)
                        l[r] = alpha * l[r] + float(np.sum(p))
                        acc[r] = alpha * acc[r] + p @ v[b, h, cols]
                        m[r] = m_new
                for r in rows:
                    o[b, h, r] = acc[r] / l[r]
                    lse[b, h, r] = m[r] + math.log(l[r])
    return o, lse
