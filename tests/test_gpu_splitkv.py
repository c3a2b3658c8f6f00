"""GPU parity of the key-split forward and of the Eq. (2) merge (through the C ABI).

``fa_fwd_splitkv`` has the contract of ``fa_fwd``, so it is held to the same
tolerances against the fp64 oracle (O max-abs 2e-2 / mean-abs 2e-3, LSE
1e-3), for automatic and explicit part counts, ragged N, both head sizes and
both mask modes, including causal grids where whole parts of a query block see
no key.  ``fa_lse_merge`` is compared with ``oracle.ref_lse_merge`` on random
fp32 parts: it computes in fp32 and rounds O once to bf16, so the bound is
2^-8 relative plus 1e-5 absolute for O, and 1e-5 (+1e-6 relative) for LSE.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from aware_exact_attention_amd.inputs import WORKLOADS, make_inputs, to_f64, workload_inputs
from test_gpu_parity import _gpu, _np, _report, check_lse, check_o, sample_rows

pytestmark = pytest.mark.gpu


def _splitkv(fa, q, k, v, causal, scale, num_splits):
    qd, kd, vd = _gpu(q, k, v)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:3], float("nan"), device="cuda", dtype=torch.float32)
    B, H, N, d = q.shape
    need = fa.splitkv_workspace_bytes(B, H, N, d, num_splits)
    ws = torch.full((max(need, 16),), 0x7F, dtype=torch.uint8, device="cuda") if need else None
    fa.fwd_splitkv(qd, kd, vd, causal=causal, scale=scale, num_splits=num_splits, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("N", [1, 100, 1000, 4097])
@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [0, 3, 7])
def test_splitkv_small(gpu_lib, N, d, causal, splits):
    q, k, v = make_inputs(1, 2, N, d, "bf16", seed=600 + N + d)
    scale = d ** -0.5
    o, lse = _splitkv(gpu_lib, q, k, v, causal, scale, splits)
    ro, rl = oracle.ref_fwd(to_f64(q), to_f64(k), to_f64(v), scale, causal)
    parts = gpu_lib.splitkv_parts(1, 2, N, d, splits)
    tag = f"splitkv N={N} d={d} causal={causal} splits={splits} parts={parts}"
    check_o(tag, _np(o), ro)
    check_lse(tag, _np(lse), rl)


@pytest.mark.parametrize("shape,causal", [((1, 8, 2048, 128), False), ((1, 4, 4096, 128), True),
                                          ((2, 3, 3000, 64), True)])
def test_splitkv_small_grids(gpu_lib, shape, causal):
    """Grids of fewer than 512 workgroups, where the automatic part count is > 1."""
    B, H, N, d = shape
    q, k, v = make_inputs(B, H, N, d, "bf16", seed=650 + N)
    scale = d ** -0.5
    parts = gpu_lib.splitkv_parts(B, H, N, d, 0)
    assert parts > 1
    o, lse = _splitkv(gpu_lib, q, k, v, causal, scale, 0)
    o, lse = _np(o), _np(lse)
    qn, kn, vn = to_f64(q), to_f64(k), to_f64(v)
    rng = np.random.default_rng(N)
    eo, el = [], []
    for b in range(B):
        for h in range(H):
            rows = sample_rows(N, rng)
            ro, rl = oracle.ref_fwd_rows(qn[b, h], kn[b, h], vn[b, h], scale, causal, rows)
            eo.append(np.abs(o[b, h, rows] - ro).ravel())
            el.append(np.abs(lse[b, h, rows] - rl))
    eo, el = np.concatenate(eo), np.concatenate(el)
    tag = f"splitkv {shape} causal={causal} parts={parts}"
    _report(check=tag, what="O(sampled rows)", max_abs=float(eo.max()), mean_abs=float(eo.mean()))
    _report(check=tag, what="LSE(sampled rows)", max_abs=float(el.max()))
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert eo.max() <= 2e-2 and eo.mean() <= 2e-3 and el.max() <= 1e-3


def test_splitkv_benchmark_shape_matches_fwd(gpu_lib):
    """At B1 H8 N2048 d128 (the pages' shortest benchmark length) the split and
    unsplit forwards agree to rounding and both meet the oracle on sampled rows."""
    w = WORKLOADS["sweep_2k"]
    q, k, v = workload_inputs(w)
    qd, kd, vd = _gpu(q, k, v)
    o1, l1 = gpu_lib.fwd(qd, kd, vd, causal=w.causal, scale=w.scale)
    o2, l2 = _splitkv(gpu_lib, q, k, v, w.causal, w.scale, 0)
    torch.cuda.synchronize()
    d_o = (o1.float() - o2.float()).abs()
    d_l = (l1 - l2).abs()
    _report(check="splitkv vs fwd sweep_2k", what="O", max_abs=float(d_o.max()), mean_abs=float(d_o.mean()))
    _report(check="splitkv vs fwd sweep_2k", what="LSE", max_abs=float(d_l.max()))
    assert float(d_o.max()) <= 2e-2 and float(d_l.max()) <= 1e-3


@pytest.mark.parametrize("S", [1, 2, 5])
@pytest.mark.parametrize("d", [64, 96, 128, 256])
def test_lse_merge(gpu_lib, S, d):
    B, H, N = 1, 3, 77
    rng = np.random.default_rng(700 + S + d)
    op = rng.normal(0.0, 1.0, size=(S, B, H, N, d)).astype(np.float32)
    lp = rng.normal(0.0, 3.0, size=(S, B, H, N)).astype(np.float32)
    if S > 1:
        lp[0, 0, 1, ::3] = -np.inf      # part 0 saw no key for some rows
        op[0, 0, 1, ::3] = 0.0
    lp[:, 0, 2, 5] = -np.inf            # a row that saw no key at all
    op[:, 0, 2, 5] = 0.0
    lp[:, 0, 0, 7] += 700.0             # large statistics must not overflow
    o, lse = gpu_lib.lse_merge(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda())
    torch.cuda.synchronize()
    o, lse = _np(o), _np(lse)
    ro, rl = oracle.ref_lse_merge(op.astype(np.float64), lp.astype(np.float64))
    assert np.all(o[0, 2, 5] == 0) and lse[0, 2, 5] == -math.inf
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin)
    eo = np.abs(o - ro)
    el = np.abs(lse[fin] - rl[fin])
    _report(check=f"lse_merge S={S} d={d}", what="O", max_abs=float(eo.max()))
    _report(check=f"lse_merge S={S} d={d}", what="LSE", max_abs=float(el.max()))
    assert np.all(eo <= 2.0 ** -8 * np.abs(ro) + 1e-5)
    assert np.all(el <= 1e-5 + 1e-6 * np.abs(rl[fin]))
