"""GPU parity of the fp16 forward and backward (fa_fwd_fp16, fa_bwd_fp16) against the fp64 oracle.

fp16 keeps 11 significant bits against bf16's 8, so the bf16 tolerances of the
other parity tests (O max-abs 2e-2 / mean-abs 2e-3, LSE 1e-3, gradients 2e-2 of
max|ref| and 1e-2 of mean|ref|) hold with room to spare; the same bounds are
used.  Inputs are the seeded N(0,1) values rounded once to fp16.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from aware_exact_attention_amd.inputs import make_inputs, to_f64
from test_gpu_parity import _gpu, _np, _report, check_grad, check_lse, check_o, sample_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N", [1, 100, 1000, 4097])
@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_fp16_forward(gpu_lib, N, d, causal):
    q, k, v = make_inputs(1, 2, N, d, "fp16", seed=1000 + N + d)
    assert q.dtype == torch.float16
    scale = d ** -0.5
    qd, kd, vd = _gpu(q, k, v)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:3], float("nan"), device="cuda", dtype=torch.float32)
    gpu_lib.fwd(qd, kd, vd, causal=causal, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.ref_fwd(to_f64(q), to_f64(k), to_f64(v), scale, causal)
    tag = f"fp16 fwd N={N} d={d} causal={causal}"
    check_o(tag, _np(out), ro)
    check_lse(tag, _np(lse), rl)


@pytest.mark.parametrize("N", [33, 300, 1000])
@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_fp16_backward(gpu_lib, N, d, causal):
    q, k, v, do = make_inputs(1, 2, N, d, "fp16", seed=1100 + N + d, backward=True)
    scale = d ** -0.5
    qd, kd, vd, dod = _gpu(q, k, v, do)
    o, lse = gpu_lib.fwd(qd, kd, vd, causal=causal, scale=scale)
    outs = tuple(torch.full_like(qd, float("nan")) for _ in range(3))
    dq, dk, dv = gpu_lib.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale, out=outs)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.ref_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, causal)
    tag = f"fp16 bwd N={N} d={d} causal={causal}"
    check_grad(tag, "dQ", _np(dq), rq)
    check_grad(tag, "dK", _np(dk), rk)
    check_grad(tag, "dV", _np(dv), rv)


def test_fp16_full_size(gpu_lib):
    """B1 H8 N16384 d128 (the benchmark shape, 8-wave forward and dQ kernels):
    forward on sampled rows of every head, backward on one full head."""
    B, H, N, d = 1, 8, 16384, 128
    q, k, v, do = make_inputs(B, H, N, d, "fp16", seed=1200, backward=True)
    scale = d ** -0.5
    qd, kd, vd, dod = _gpu(q, k, v, do)
    o, lse = gpu_lib.fwd(qd, kd, vd, scale=scale)
    dq, dk, dv = gpu_lib.bwd(qd, kd, vd, o, lse, dod, scale=scale)
    torch.cuda.synchronize()
    on, ln = _np(o), _np(lse)
    qn, kn, vn, don = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    rng = np.random.default_rng(1200)
    eo, el = [], []
    for h in range(H):
        rows = sample_rows(N, rng, extra=96)
        ro, rl = oracle.ref_fwd_rows(qn[0, h], kn[0, h], vn[0, h], scale, False, rows)
        eo.append(np.abs(on[0, h, rows] - ro).ravel())
        el.append(np.abs(ln[0, h, rows] - rl))
    eo, el = np.concatenate(eo), np.concatenate(el)
    _report(check="fp16 full size", what="O(sampled rows)", max_abs=float(eo.max()), mean_abs=float(eo.mean()))
    assert eo.max() <= 2e-2 and eo.mean() <= 2e-3 and el.max() <= 1e-3
    h = 3
    sl = (slice(0, 1), slice(h, h + 1))
    rq, rk, rv = oracle.ref_bwd(qn[sl], kn[sl], vn[sl], don[sl], scale, False)
    check_grad("fp16 full size head 3", "dQ", _np(dq)[sl], rq)
    check_grad("fp16 full size head 3", "dK", _np(dk)[sl], rk)
    check_grad("fp16 full size head 3", "dV", _np(dv)[sl], rv)
