"""GPU parity of the forward and backward with dropout (fa_fwd_dropout, fa_bwd_dropout).

The kernels draw the keep mask in place (Philox4x32-10, one call per 4 x 4
block of P) and the oracle (``oracle/dropout.py``) draws the same mask from the
same definition; the outputs are then held to the bf16 tolerances of the other
parity tests.  With p = 0 every element is kept and scaled by exactly 1, so the
dropout forward must equal ``fa_fwd`` bit for bit.
"""
from __future__ import annotations

import pytest
import torch

import oracle
from aware_exact_attention_amd.inputs import make_inputs, to_f64
from test_gpu_parity import _gpu, _np, check_grad, check_lse, check_o

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N", [1, 100, 1000, 2049])
@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.1, 0.5])
def test_dropout_forward(gpu_lib, N, d, causal, p):
    q, k, v = make_inputs(1, 2, N, d, "bf16", seed=1300 + N + d)
    scale, seed = d ** -0.5, 0x1234_5678_9ABC + N
    qd, kd, vd = _gpu(q, k, v)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:3], float("nan"), device="cuda", dtype=torch.float32)
    gpu_lib.fwd_dropout(qd, kd, vd, p, seed, causal=causal, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.ref_fwd_dropout(to_f64(q), to_f64(k), to_f64(v), scale, causal, p, seed)
    tag = f"dropout fwd N={N} d={d} causal={causal} p={p}"
    check_o(tag, _np(out), ro)
    check_lse(tag, _np(lse), rl)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_p0_equals_plain(gpu_lib, causal):
    # a grid that fills the GPU, where the plain forward also gives each row
    # to one wave (on small grids it splits a row's keys over several waves,
    # which sums in another order)
    q, k, v = _gpu(*make_inputs(4, 16, 777, 128, "bf16", seed=1350))
    o1, l1 = gpu_lib.fwd(q, k, v, causal=causal)
    o2, l2 = gpu_lib.fwd_dropout(q, k, v, 0.0, 99, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("N", [33, 300, 1000])
@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.1, 0.3])
def test_dropout_backward(gpu_lib, N, d, causal, p):
    q, k, v, do = make_inputs(1, 2, N, d, "bf16", seed=1400 + N + d, backward=True)
    scale, seed = d ** -0.5, 0xDEAD_BEEF_0000 + N
    qd, kd, vd, dod = _gpu(q, k, v, do)
    o, lse = gpu_lib.fwd_dropout(qd, kd, vd, p, seed, causal=causal, scale=scale)
    outs = tuple(torch.full_like(qd, float("nan")) for _ in range(3))
    dq, dk, dv = gpu_lib.bwd_dropout(qd, kd, vd, o, lse, dod, p, seed, causal=causal, scale=scale, out=outs)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.ref_bwd_dropout(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, causal, p, seed)
    tag = f"dropout bwd N={N} d={d} causal={causal} p={p}"
    check_grad(tag, "dQ", _np(dq), rq)
    check_grad(tag, "dK", _np(dk), rk)
    check_grad(tag, "dV", _np(dv), rv)


def test_dropout_larger(gpu_lib):
    """B1 H2 N4096 d128 (four-wave forward) and B1 H64 N2048 d128 (eight-wave
    forward and dQ kernels, persistent dK/dV workgroups), dense and causal, at
    p = 0.1, compared on the last head."""
    for (B, H, N, causal) in ((1, 2, 4096, False), (1, 64, 2048, False), (1, 64, 2048, True)):
        q, k, v, do = make_inputs(B, H, N, 128, "bf16", seed=1500 + H, backward=True)
        scale, seed, p = 128 ** -0.5, 4242, 0.1
        qd, kd, vd, dod = _gpu(q, k, v, do)
        o, lse = gpu_lib.fwd_dropout(qd, kd, vd, p, seed, causal=causal, scale=scale)
        dq, dk, dv = gpu_lib.bwd_dropout(qd, kd, vd, o, lse, dod, p, seed, causal=causal, scale=scale)
        torch.cuda.synchronize()
        h = H - 1
        sl = (slice(0, 1), slice(h, h + 1))
        args = [to_f64(t[sl]) for t in (q, k, v, do)]
        ro, rl = oracle.ref_fwd_dropout(*args[:3], scale, causal, p, seed, bh0=h)
        rq, rk, rv = oracle.ref_bwd_dropout(*args, scale, causal, p, seed, bh0=h)
        tag = f"dropout B{B} H{H} N{N} causal={causal} head {h}"
        check_o(tag, _np(o)[sl], ro)
        check_lse(tag, _np(lse)[sl], rl)
        check_grad(tag, "dQ", _np(dq)[sl], rq)
        check_grad(tag, "dK", _np(dk)[sl], rk)
        check_grad(tag, "dV", _np(dv)[sl], rv)
