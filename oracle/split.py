"""fp64 oracle for attention split over key ranges and the merge of the parts.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle/ref.py``: only tests, the smoke
check and the CPU-baseline leg of the benchmark may use it; it shares nothing
with the HIP library).

Eq. (2) of the Journal of Software 2026(1) p.218 LLM pre-training survey says
how the softmax statistics of two blocks of a row combine: with ``(m1, l1)`` and
``(m2, l2)`` the block maxima and block sums of ``exp(x - m)``, the whole row
has ``m = max(m1, m2)`` and ``l = e^(m1-m) l1 + e^(m2-m) l2``, and each block's
exponentials are rescaled by its factor ``e^(mi-m)``.  Applied to attention, a
row's keys can be cut into ranges, each range gives a normalised partial output
``O_s = sum_j p_j v_j / l_s`` and the statistic ``LSE_s = m_s + ln l_s``, and the
full result is recovered from the parts alone:

* the factor of part s relative to the whole row is
  ``e^(m_s-m) l_s / l = e^(LSE_s - LSE)``, where ``LSE = ln sum_s e^(LSE_s)``;
* ``O = sum_s e^(LSE_s - LSE) O_s``.

``ref_lse_merge`` computes exactly this, subtracting the largest ``LSE_s``
before exponentiating (the same safe-softmax device as Eq. (1)).  A part whose
row saw no key at all has ``l_s = 0``, i.e. ``LSE_s = -inf``; its factor is 0
(the limit of Eq. (2)) and its ``O_s`` is ignored.

``ref_fwd_keyrange`` is the plain definition restricted to the keys
``k0 <= j < k1`` (plus the causal mask ``j <= i`` on absolute positions), so that
a test can split the keys of one attention call any way it likes.
"""
from __future__ import annotations

import numpy as np

from .ref import _as_f64, _scores


def ref_fwd_keyrange(q, k, v, scale: float, causal: bool, k0: int, k1: int):
    """Attention of every query over keys ``k0 <= j < k1`` only.

    Returns ``(O_part [B,H,N,d], LSE_part [B,H,N])`` in float64.  A row with no
    visible key in the range gets ``O = 0`` and ``LSE = -inf``.
    """
    q, k, v = _as_f64(q, k, v)
    B, H, N, _ = q.shape
    o = np.zeros((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.full((B, H, N), -np.inf, dtype=np.float64)
    outside = np.ones(k.shape[2], dtype=bool)
    outside[max(k0, 0):max(k1, 0)] = False
    for b in range(B):
        for h in range(H):
            s = _scores(q[b, h], k[b, h], scale, causal)
            s[:, outside] = -np.inf
            m = s.max(axis=1)
            seen = m > -np.inf
            if not seen.any():
                continue
            f = np.exp(s[seen] - m[seen, None])
            l = f.sum(axis=1)
            o[b, h, seen] = (f @ v[b, h]) / l[:, None]
            lse[b, h, seen] = m[seen] + np.log(l)
    return o, lse


def ref_lse_merge(o_parts, lse_parts):
    """Eq. (2) over S parts: ``o_parts [S,B,H,N,d]``, ``lse_parts [S,B,H,N]``.

    Returns ``(O [B,H,N,d], LSE [B,H,N])`` in float64.  Rows where every part is
    ``-inf`` get ``O = 0`` and ``LSE = -inf``.
    """
    o_parts, lse_parts = _as_f64(o_parts, lse_parts)
    top = lse_parts.max(axis=0)  # [B,H,N]
    finite = top > -np.inf
    ref = np.where(finite, top, 0.0)
    w = np.where(lse_parts > -np.inf, np.exp(lse_parts - ref[None]), 0.0)  # e^(LSE_s - max)
    total = w.sum(axis=0)
    safe = np.where(finite, total, 1.0)
    o = (w[..., None] * np.where(w[..., None] > 0, o_parts, 0.0)).sum(axis=0) / safe[..., None]
    lse = np.where(finite, ref + np.log(safe), -np.inf)
    return o, lse
