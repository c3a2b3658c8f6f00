"""fp64 oracle for attention with dropout on the probabilities.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle/ref.py``).

The Journal of Software survey (the sentence after Eq. (2) on what the fused
kernel does) lists dropout among the operations fused into one kernel; the
pages give no random-number scheme.  The reading written out here:

* The random bits come from Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
  "Parallel random numbers: as easy as 1, 2, 3", SC 2011): a counter-based
  generator, so the GPU kernels (forward and backward) and this oracle can each
  compute the bits of any element independently.  One call maps a 128-bit
  counter (c0, c1, c2, c3) and a 64-bit key (k0, k1) through ten rounds; a round
  multiplies c0 and c2 by the constants 0xD2511F53 and 0xCD9E8D57 into 64-bit
  products (hi, lo) and returns ``(hi(c2*M1) ^ c1 ^ k0, lo(c2*M1),
  hi(c0*M0) ^ c3 ^ k1, lo(c0*M0))``; between rounds the key is bumped by the
  Weyl constants 0x9E3779B9 and 0xBB67AE85.
* Element (b, h, i, j) of the probability matrix belongs to the 4 x 4 block
  (i // 4, j // 4).  Its call has counter ``(i // 4, j // 4, b*H + h, 0)`` and key
  ``(seed mod 2^32, seed // 2^32)``; of the four 32-bit outputs, word ``i % 4``
  holds the block's row i, and its byte ``j % 4`` (little-endian) is the
  element's 8-bit draw u in [0, 255].
* With drop probability p, the threshold is ``t = round(256 p)`` (0 <= t <= 255);
  the element is kept iff ``u >= t``, so the effective drop probability is
  ``t / 256``, and kept probabilities are scaled by ``1 / (1 - t/256)``.
* Forward: ``O = (P * Z) V`` with ``Z = keep / (1 - t/256)``; the statistic
  LSE is that of the softmax before dropout.
* Backward: ``dV = (P*Z)^T dO``, ``dP = (dO V^T) * Z``, ``D_i = sum_j P_ij dP_ij``
  (equal to ``sum_k dO_ik O_ik``), ``dS = P * (dP - D)``, ``dQ = scale dS K``,
  ``dK = scale dS^T Q``: the chain rule on the forward above.
"""
from __future__ import annotations

import numpy as np

from .ref import _as_f64, _scores, _softmax_rows

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32(c0, c1, c2, c3, k0, k1, rounds: int = 10):
    """Philox4x32 on numpy uint64 arrays holding 32-bit values (broadcast); returns 4 arrays."""
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & MASK32 for x in (c0, c1, c2, c3))
    k0 = np.uint64(int(k0) & MASK32)
    k1 = np.uint64(int(k1) & MASK32)
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    sh, m32 = np.uint64(32), np.uint64(MASK32)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & m32
            k1 = (k1 + np.uint64(PHILOX_W1)) & m32
        p0 = c0 * m0  # < 2^64: exact in uint64
        p1 = c2 * m1
        c0, c1, c2, c3 = ((p1 >> sh) ^ c1 ^ k0), (p1 & m32), ((p0 >> sh) ^ c3 ^ k1), (p0 & m32)
    return c0, c1, c2, c3


def threshold(p: float) -> int:
    """8-bit drop threshold t = round(256 p), clamped to [0, 255]."""
    return int(min(255, max(0, int(np.floor(256.0 * p + 0.5)))))


def keep_mask_bh(N: int, bh: int, seed: int, p: float) -> np.ndarray:
    """``[N, N]`` bool keep mask of the head whose counter word is ``bh`` (= b*H + h)."""
    t = threshold(p)
    i = np.broadcast_to(np.arange(N)[:, None], (N, N))  # query index
    j = np.broadcast_to(np.arange(N)[None, :], (N, N))  # key index
    words = np.stack(philox4x32(i // 4, j // 4, np.full((N, N), bh), np.zeros((N, N)),
                                seed & MASK32, seed >> 32))            # [4, N, N]
    w = np.take_along_axis(words, (i % 4)[None], axis=0)[0]           # word i % 4
    u = (w >> (8 * (j % 4)).astype(np.uint64)) & np.uint64(0xFF)      # byte j % 4
    return u >= t


def keep_mask(B: int, H: int, N: int, seed: int, p: float, bh0: int = 0) -> np.ndarray:
    """``[B,H,N,N]`` bool: element (b, h, i, j) kept, with head counter ``bh0 + b*H + h``.

    ``bh0`` lets a caller evaluate a slice of heads of a larger tensor (for
    B = 1, head h of an H-head tensor is ``keep_mask(1, 1, N, seed, p, bh0=h)``).
    """
    out = np.empty((B, H, N, N), dtype=bool)
    for b in range(B):
        for h in range(H):
            out[b, h] = keep_mask_bh(N, bh0 + b * H + h, seed, p)
    return out


def dropout_scale(p: float) -> float:
    return 1.0 / (1.0 - threshold(p) / 256.0)


def ref_fwd_dropout(q, k, v, scale: float, causal: bool, p: float, seed: int, bh0: int = 0):
    """``(O, LSE)`` with dropout on P; LSE is the pre-dropout statistic (``bh0`` as in keep_mask)."""
    q, k, v = _as_f64(q, k, v)
    B, H, N, _ = q.shape
    z = keep_mask(B, H, N, seed, p, bh0) * dropout_scale(p)
    o = np.empty((B, H, N, v.shape[-1]))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            P, m, l = _softmax_rows(_scores(q[b, h], k[b, h], scale, causal))
            o[b, h] = (P * z[b, h]) @ v[b, h]
            lse[b, h] = m + np.log(l)
    return o, lse


def ref_bwd_dropout(q, k, v, do, scale: float, causal: bool, p: float, seed: int, bh0: int = 0):
    """Gradients ``(dQ, dK, dV)`` of ``sum(O * dO)`` for the dropout forward above."""
    q, k, v, do = _as_f64(q, k, v, do)
    B, H, N, _ = q.shape
    z = keep_mask(B, H, N, seed, p, bh0) * dropout_scale(p)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(B):
        for h in range(H):
            P = _softmax_rows(_scores(q[b, h], k[b, h], scale, causal))[0]
            dv[b, h] = (P * z[b, h]).T @ do[b, h]
            dp = (do[b, h] @ v[b, h].T) * z[b, h]
            D = (P * dp).sum(axis=1, keepdims=True)
            ds = P * (dp - D)
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv
