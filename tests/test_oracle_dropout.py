"""Pins of the dropout oracle (``oracle/dropout.py``).

Philox4x32-10 (Salmon et al., SC 2011) is pinned by special cases of its
definition that expose each constant and the word order, by determinism and by
the uniformity of its bytes; the dropout attention is pinned by p = 0 (plain
attention, itself pinned in ``test_oracle.py``), by the keep rate, by central
finite differences of the backward with the mask held fixed, and by
torch.autograd on plain fp64 ops with the same mask.

The full 10-round stream is pinned against an independent implementation:
rocRAND's open-source Philox4x32-10 engine (``rocrand/rocrand_philox4x32_10.h``
of the ROCm install, host-callable), compiled with g++ into a small host
program and compared word for word on random (counter, key) pairs.

What is a reading and not pinned by anything outside this build: the mapping of
(b, h, i, j) to counters, words and bytes (a convention both sides implement).
"""
from __future__ import annotations

import functools
import math
import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle.dropout as dropout_module
import oracle.ref as ref_module


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).normal(0.0, std, size=shape)


def pin_philox_one_round(R):
    # c0 = c2 = 1: the products are the multipliers themselves (hi = 0, lo = M)
    for c1, c3, k0, k1 in ((0, 0, 0, 0), (0x12345678, 0x9ABCDEF0, 0x0F0F0F0F, 0xF0F0F0F0)):
        w = [int(x) for x in R.philox4x32(1, c1, 1, c3, k0, k1, rounds=1)]
        assert w == [c1 ^ k0, 0xCD9E8D57, c3 ^ k1, 0xD2511F53]
    # c0 = 2^31: lo = 0 or 2^31, hi = M >> 1 (a shift of the 64-bit product)
    w = [int(x) for x in R.philox4x32(1 << 31, 0, 1 << 31, 0, 0, 0, rounds=1)]
    assert w == [0xCD9E8D57 >> 1, (0xCD9E8D57 << 31) & 0xFFFFFFFF, 0xD2511F53 >> 1, (0xD2511F53 << 31) & 0xFFFFFFFF]


def pin_philox_key_schedule(R):
    # key = (c1, c3) and c0 = c2 = 0 zero the first round; the second round then
    # returns the bumped key: (k0 + W0, 0, k1 + W1, 0)
    for k0, k1 in ((0, 0), (5, 7), (0xFFFFFFFF, 0x80000000)):
        w = [int(x) for x in R.philox4x32(0, k0, 0, k1, k0, k1, rounds=2)]
        assert w == [(k0 + 0x9E3779B9) & 0xFFFFFFFF, 0, (k1 + 0xBB67AE85) & 0xFFFFFFFF, 0]


def pin_philox_statistics(R):
    n = 1 << 16
    c = np.arange(n)
    w = R.philox4x32(c, 0, 7, 0, 0x1234, 0x5678)
    a = [int(x) for x in R.philox4x32(c[:3], 0, 7, 0, 0x1234, 0x5678)[0]]
    assert a == [int(x) for x in w[0][:3]]  # deterministic
    b = np.concatenate([(x[:, None] >> (8 * np.arange(4, dtype=np.uint64))) & np.uint64(0xFF) for x in w]).ravel()
    hist = np.bincount(b.astype(np.int64), minlength=256)
    exp = b.size / 256
    chi2 = float(((hist - exp) ** 2 / exp).sum())
    assert chi2 < 400, chi2  # 255 degrees of freedom: mean 255, sd 22.6
    # one seed bit changes about half of the output bits
    w2 = R.philox4x32(c, 0, 7, 0, 0x1235, 0x5678)
    flips = sum(int(np.unpackbits((x ^ y).astype(">u4").view(np.uint8)).sum()) for x, y in zip(w, w2))
    assert abs(flips / (n * 128) - 0.5) < 0.01


def pin_p_zero_is_plain(R):
    q, k, v, do = (_rand((1, 2, 23, 8), 300 + i) for i in range(4))
    for causal in (False, True):
        o, lse = R.ref_fwd_dropout(q, k, v, 0.4, causal, 0.0, 99)
        ro, rl = ref_module.ref_fwd(q, k, v, 0.4, causal)
        np.testing.assert_allclose(o, ro, rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-14)
        g = R.ref_bwd_dropout(q, k, v, do, 0.4, causal, 0.0, 99)
        rg = ref_module.ref_bwd(q, k, v, do, 0.4, causal)
        for a, b in zip(g, rg):
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def pin_keep_rate(R):
    for p in (0.1, 0.5, 0.9):
        m = R.keep_mask(1, 2, 512, 2024, p)
        t = R.threshold(p)
        keep = 1 - t / 256
        sd = math.sqrt(keep * (1 - keep) / m.size)
        assert abs(m.mean() - keep) < 5 * sd, (p, m.mean(), keep)
        # a different seed or head gives a different mask
        assert (m[0, 0] != m[0, 1]).mean() > 0.1
        # a slice of heads evaluated on its own sees the same mask
        assert np.array_equal(R.keep_mask(1, 1, 512, 2024, p, bh0=1)[0, 0], m[0, 1])
    assert R.threshold(0.0) == 0 and R.threshold(0.5) == 128 and R.threshold(0.999) == 255
    assert abs(R.dropout_scale(0.5) - 2.0) < 1e-15


def _loss(R, q, k, v, do, scale, causal, p, seed):
    return float((R.ref_fwd_dropout(q, k, v, scale, causal, p, seed)[0] * do).sum())


def pin_finite_differences(R):
    N, d, scale, eps, p, seed = 8, 3, 0.7, 1e-6, 0.3, 5
    q, k, v, do = (_rand((1, 1, N, d), 310 + i) for i in range(4))
    assert not R.keep_mask(1, 1, N, seed, p).all()  # some elements are dropped
    for causal in (False, True):
        grads = R.ref_bwd_dropout(q, k, v, do, scale, causal, p, seed)
        for which, g in enumerate(grads):
            num = np.zeros_like(g)
            for idx in np.ndindex(*g.shape):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][idx] += eps
                lp = _loss(R, *args, do, scale, causal, p, seed)
                args[which][idx] -= 2 * eps
                lm = _loss(R, *args, do, scale, causal, p, seed)
                num[idx] = (lp - lm) / (2 * eps)
            np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def pin_autograd(R):
    B, H, N, d, scale, p, seed = 1, 2, 12, 5, 0.45, 0.25, 77
    arrs = [_rand((B, H, N, d), 320 + i) for i in range(4)]
    z = torch.from_numpy(R.keep_mask(B, H, N, seed, p) * R.dropout_scale(p))
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in arrs[:3])
        s = scale * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
        o = (torch.softmax(s, -1) * z) @ tv
        (o * torch.from_numpy(arrs[3])).sum().backward()
        of, _ = R.ref_fwd_dropout(*arrs[:3], scale, causal, p, seed)
        np.testing.assert_allclose(of, o.detach().numpy(), rtol=0, atol=1e-13)
        dq, dk, dv = R.ref_bwd_dropout(*arrs, scale, causal, p, seed)
        np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-13)
        np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-13)


ROCRAND_HEADER = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
# Host program around rocRAND's engine: reads "c0 c1 c2 c3 k0 k1" lines and
# prints the four words of the 10-round block function.  The block function
# is a protected member of the engine; a derived class exposes it.  The
# engine's public seeding path (seed -> key, subsequence -> (c2, c3),
# offset / 4 -> (c0, c1)) is printed beside it for the small counters where
# that path can express the counter (4 * (c1:c0) < 2^64).
_ROCRAND_PROBE = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
struct Probe : rocrand_device::philox4x32_10_engine {
  uint4 block(uint4 c, uint2 k) { return ten_rounds(c, k); }
};
int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  Probe p;
  while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint4 c; c.x = c0; c.y = c1; c.z = c2; c.w = c3;
    uint2 k; k.x = k0; k.y = k1;
    const uint4 w = p.block(c, k);
    unsigned e[4] = {0, 0, 0, 0};
    if (c1 < (1u << 30)) {
      rocrand_device::philox4x32_10_engine g((unsigned long long)k1 << 32 | k0,
                                             (unsigned long long)c3 << 32 | c2,
                                             4ull * ((unsigned long long)c1 << 32 | c0));
      for (int i = 0; i < 4; ++i) e[i] = g();
    }
    std::printf("%u %u %u %u %u %u %u %u\n", w.x, w.y, w.z, w.w, e[0], e[1], e[2], e[3]);
  }
  return 0;
}
"""


@functools.lru_cache(maxsize=1)
def _rocrand_probe() -> str:
    d = tempfile.mkdtemp(prefix="philox_rocrand_")
    src, exe = os.path.join(d, "probe.cpp"), os.path.join(d, "probe")
    with open(src, "w") as f:
        f.write(_ROCRAND_PROBE)
    subprocess.run(["g++", "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", src, "-o", exe],
                   check=True, capture_output=True, text=True)
    return exe


def _rocrand_words(ctr: np.ndarray, key: np.ndarray):
    """rocRAND's 10-round outputs for rows (c0, c1, c2, c3) and (k0, k1): block words, engine words."""
    lines = "\n".join(" ".join(str(int(x)) for x in (*c, *k)) for c, k in zip(ctr, key)) + "\n"
    out = subprocess.run([_rocrand_probe()], input=lines, capture_output=True, text=True, check=True).stdout
    vals = np.array([[int(x) for x in ln.split()] for ln in out.strip().splitlines()], dtype=np.uint64)
    return vals[:, :4], vals[:, 4:]


def pin_philox_rocrand(R):
    """Ten rounds against rocRAND's Philox4x32-10, word for word: 40 random keys
    with 300 random counters each (full 32-bit range; a third of them small, as
    the dropout mask uses, a third with c1 < 2^30 so that the engine's public
    seeding path applies), plus the all-zero and all-ones cases."""
    if not os.path.exists(ROCRAND_HEADER):
        raise AssertionError(f"{ROCRAND_HEADER} missing: the 10-round pin cannot run")
    rng = np.random.default_rng(20260101)
    nk, nc = 40, 300
    keys = rng.integers(0, 1 << 32, size=(nk, 2), dtype=np.uint64)
    keys[0] = 0
    keys[1] = 0xFFFFFFFF
    ctr = rng.integers(0, 1 << 32, size=(nk, nc, 4), dtype=np.uint64)
    ctr[:, : nc // 3, 1] &= (1 << 30) - 1
    ctr[:, nc // 3: 2 * nc // 3, 1:] = 0
    ctr[:, nc // 3: 2 * nc // 3, 0] &= 0xFFFF
    ctr[0, 0] = 0
    ctr[1, 0] = 0xFFFFFFFF
    flat_c = ctr.reshape(-1, 4)
    flat_k = np.repeat(keys, nc, axis=0)
    block, engine = _rocrand_words(flat_c, flat_k)
    got = np.empty_like(block)
    for i in range(nk):
        w = R.philox4x32(*(ctr[i, :, j] for j in range(4)), int(keys[i, 0]), int(keys[i, 1]))
        got[i * nc:(i + 1) * nc] = np.stack([np.asarray(x, dtype=np.uint64) for x in w], axis=1)
    bad = np.nonzero((got != block).any(axis=1))[0]
    assert bad.size == 0, (f"{bad.size} of {len(flat_c)} blocks differ from rocRAND "
                           f"(first: counter {flat_c[bad[0]]}, key {flat_k[bad[0]]})")
    seeded = flat_c[:, 1] < (1 << 30)
    assert seeded.sum() > nk * nc // 3
    assert np.array_equal(engine[seeded], block[seeded]), "rocRAND's seeding path disagrees with its block function"


PINS = [pin_philox_one_round, pin_philox_key_schedule, pin_philox_statistics, pin_philox_rocrand,
        pin_p_zero_is_plain, pin_keep_rate, pin_finite_differences, pin_autograd]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_dropout_oracle_pin(pin):
    pin(dropout_module)


_ORIG_PHILOX = dropout_module.philox4x32
_ORIG_BWD = dropout_module.ref_bwd_dropout
_ORIG_SCALE = dropout_module.dropout_scale


def _mut_philox_words_swapped(c0, c1, c2, c3, k0, k1, rounds=10):
    a, b, c, d = _ORIG_PHILOX(c0, c1, c2, c3, k0, k1, rounds)
    return c, b, a, d


def _mut_philox_no_key_bump(c0, c1, c2, c3, k0, k1, rounds=10):
    out = (c0, c1, c2, c3)
    for _ in range(rounds):
        out = _ORIG_PHILOX(*out, k0, k1, rounds=1)
    return out


# A stream of 9 or 7 rounds whose round function is right: the one- and
# two-round special cases still hold, so only the rocRAND pin sees it.
def _mut_philox_9_rounds(c0, c1, c2, c3, k0, k1, rounds=10):
    return _ORIG_PHILOX(c0, c1, c2, c3, k0, k1, 9 if rounds == 10 else rounds)


def _mut_philox_7_rounds(c0, c1, c2, c3, k0, k1, rounds=10):
    return _ORIG_PHILOX(c0, c1, c2, c3, k0, k1, 7 if rounds == 10 else rounds)


def _mut_bwd_unmasked_dp(q, k, v, do, scale, causal, p, seed):
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    B, H, N, _ = q.shape
    z = dropout_module.keep_mask(B, H, N, seed, p) * _ORIG_SCALE(p)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(B):
        for h in range(H):
            P = ref_module._softmax_rows(ref_module._scores(q[b, h], k[b, h], scale, causal))[0]
            dv[b, h] = (P * z[b, h]).T @ do[b, h]
            dp = do[b, h] @ v[b, h].T  # mask not applied
            ds = P * (dp - (P * dp).sum(axis=1, keepdims=True))
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv


def _mut_no_rescale(p):
    return 1.0


MUTANTS = {
    "philox_words_swapped": ("philox4x32", _mut_philox_words_swapped),
    "philox_no_key_bump": ("philox4x32", _mut_philox_no_key_bump),
    "philox_9_rounds": ("philox4x32", _mut_philox_9_rounds),
    "philox_7_rounds": ("philox4x32", _mut_philox_7_rounds),
    "bwd_unmasked_dp": ("ref_bwd_dropout", _mut_bwd_unmasked_dp),
    "no_rescale_of_kept": ("dropout_scale", _mut_no_rescale),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_dropout_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(dropout_module, attr, fn)
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(dropout_module)
            except (AssertionError, FloatingPointError, ValueError, TypeError):
                caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
