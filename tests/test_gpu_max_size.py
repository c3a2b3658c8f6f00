"""GPU parity at the longest sequence the API accepts for d = 128: N = 4194047, causal, one head, bf16.

(N + 256) * d * 4 < 2^31 is the bound on one head's fp32 slab addressed with 32-bit byte offsets, so this case
puts the kernels' 32-bit offsets and buffer sizes at the edge the validation allows.  The forward is compared with
the fp64 oracle on sampled rows (first, last, around a power of two, random).  For the backward, dQ is compared
on the last 16 rows.  dK and dV are compared on the last 16 keys: under the causal mask only those rows see those
keys, so the oracle's row-subset sums there are complete.  Tolerances are those of the other parity tests.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from aware_exact_attention_amd.inputs import make_inputs, to_f64
from test_gpu_parity import _gpu, _np, check_grad, check_lse, check_o

pytestmark = pytest.mark.gpu

N_MAX_D128 = 4194047  # largest N with (N + 256) * 128 * 4 < 2^31


def test_max_length_causal_d128(gpu_lib):
    assert (N_MAX_D128 + 256) * 128 * 4 < 2 ** 31 <= (N_MAX_D128 + 257) * 128 * 4
    N, d = N_MAX_D128, 128
    scale = d ** -0.5
    q, k, v, do = make_inputs(1, 1, N, d, "bf16", seed=1500, backward=True)
    qd, kd, vd, dod = _gpu(q, k, v, do)
    o, lse = gpu_lib.fwd(qd, kd, vd, causal=True, scale=scale)
    dq, dk, dv = gpu_lib.bwd(qd, kd, vd, o, lse, dod, causal=True, scale=scale)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t).all().item()
    rng = np.random.default_rng(1501)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(N - 8, N), [2 ** 21 - 1, 2 ** 21, 2 ** 21 + 1],
                                     rng.choice(N, size=9, replace=False)]))
    tail = np.arange(N - 16, N)
    ri, ti = torch.from_numpy(rows).cuda(), torch.from_numpy(tail).cuda()
    o_r, lse_r = _np(o[0, 0, ri]), _np(lse[0, 0, ri])
    dq_t, dk_t, dv_t = (_np(t[0, 0, ti]) for t in (dq, dk, dv))
    del qd, kd, vd, dod, o, lse, dq, dk, dv
    torch.cuda.empty_cache()

    qn, kn, vn, don = (to_f64(t)[0, 0] for t in (q, k, v, do))
    ro, rl = oracle.ref_fwd_rows(qn, kn, vn, scale, True, rows)
    check_o("max length fwd", o_r, ro)
    check_lse("max length fwd", lse_r, rl)
    rq, rk, rv = oracle.ref_bwd_rows(qn, kn, vn, don, scale, True, tail, tail)
    check_grad("max length bwd (last 16 rows / keys)", "dQ", dq_t, rq)
    check_grad("max length bwd (last 16 rows / keys)", "dK", dk_t, rk)
    check_grad("max length bwd (last 16 rows / keys)", "dV", dv_t, rv)
