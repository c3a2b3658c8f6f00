"""GPU parity of the float16 key split, merge, masks and dropout (the ``*_fp16`` entry points).

Each has the contract of its bf16 counterpart with float16 tensors, so the same
fp64 oracles and the same tolerances apply (float16 rounds P, dS and the outputs
at 2^-11 relative, finer than bf16's 2^-8).  The inputs are the seeded bf16
workloads' generator with one RNE conversion to float16 instead.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from aware_exact_attention_amd.inputs import make_inputs, to_f64
from test_gpu_masks import _random_block_mask
from test_gpu_masks_bwd import _check3, _check_blocks
from test_gpu_parity import _gpu, _np, check_lse, check_o

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N", [300, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window", [(5, 3), (100, 0), (-1, 0), (0, -1)], ids=["5_3", "100_0", "m1_0", "0_m1"])
def test_window_fp16(gpu_lib, N, d, window):
    left, right = window
    q, k, v, do = make_inputs(1, 2, N, d, "fp16", seed=1600 + N + d, backward=True)
    scale = d ** -0.5
    qd, kd, vd, dod = _gpu(q, k, v, do)
    o, lse = gpu_lib.fwd_window(qd, kd, vd, left, right, scale=scale)
    assert o.dtype == torch.float16
    g = gpu_lib.bwd_window(qd, kd, vd, o, lse, dod, left, right, scale=scale)
    torch.cuda.synchronize()
    args = [to_f64(t) for t in (q, k, v, do)]
    ro, rl = oracle.ref_fwd_window(*args[:3], scale, left, right)
    tag = f"fp16 window N={N} d={d} ({left},{right})"
    check_o(tag, _np(o), ro)
    check_lse(tag, _np(lse), rl)
    _check3(tag, tuple(_np(t) for t in g), oracle.ref_bwd_window(*args, scale, left, right))


@pytest.mark.parametrize("N", [130, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_fp16(gpu_lib, N, causal):
    H, d = 3, 128
    q, k, v, do = make_inputs(1, H, N, d, "fp16", seed=1700 + N, backward=True)
    scale = d ** -0.5
    bm = _random_block_mask(H, (N + 63) // 64, 0.5, N + int(causal), per_head=True)
    qd, kd, vd, dod = _gpu(q, k, v, do)
    m = torch.from_numpy(bm).cuda()
    o, lse = gpu_lib.fwd_blocksparse(qd, kd, vd, m, causal=causal, scale=scale)
    g = gpu_lib.bwd_blocksparse(qd, kd, vd, o, lse, dod, m, causal=causal, scale=scale)
    torch.cuda.synchronize()
    args = [to_f64(t) for t in (q, k, v, do)]
    ro, rl = oracle.ref_fwd_blocksparse(*args[:3], scale, causal, bm)
    o, lse = _np(o), _np(lse)
    empty = np.isinf(rl)
    assert np.array_equal(np.isinf(lse), empty) and np.all(o[empty] == 0)
    tag = f"fp16 blocksparse N={N} causal={causal}"
    check_o(tag, o[~empty], ro[~empty])
    check_lse(tag, lse[~empty], rl[~empty])
    _check_blocks(tag, tuple(_np(t) for t in g), oracle.ref_bwd_blocksparse(*args, scale, causal, bm), bm, causal, N)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_fp16(gpu_lib, causal):
    N, d, p, seed = 777, 128, 0.2, 0xABCDEF
    q, k, v, do = make_inputs(1, 2, N, d, "fp16", seed=1800, backward=True)
    scale = d ** -0.5
    qd, kd, vd, dod = _gpu(q, k, v, do)
    o, lse = gpu_lib.fwd_dropout(qd, kd, vd, p, seed, causal=causal, scale=scale)
    g = gpu_lib.bwd_dropout(qd, kd, vd, o, lse, dod, p, seed, causal=causal, scale=scale)
    torch.cuda.synchronize()
    args = [to_f64(t) for t in (q, k, v, do)]
    ro, rl = oracle.ref_fwd_dropout(*args[:3], scale, causal, p, seed)
    tag = f"fp16 dropout causal={causal}"
    check_o(tag, _np(o), ro)
    check_lse(tag, _np(lse), rl)
    _check3(tag, tuple(_np(t) for t in g), oracle.ref_bwd_dropout(*args, scale, causal, p, seed))


@pytest.mark.parametrize("N", [1000, 4097])
@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_and_merge_fp16(gpu_lib, N, causal):
    d = 128
    q, k, v = make_inputs(1, 2, N, d, "fp16", seed=1900 + N)
    scale = d ** -0.5
    qd, kd, vd = _gpu(q, k, v)
    o, lse = gpu_lib.fwd_splitkv(qd, kd, vd, causal=causal, scale=scale, num_splits=3)
    o1, l1 = gpu_lib.fwd(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    ro, rl = oracle.ref_fwd(to_f64(q), to_f64(k), to_f64(v), scale, causal)
    check_o(f"fp16 splitkv N={N} causal={causal}", _np(o), ro)
    check_lse(f"fp16 splitkv N={N} causal={causal}", _np(lse), rl)
    # the merge alone, float16 output, on fp32 parts
    S, rng = 3, np.random.default_rng(N)
    op = rng.normal(0.0, 1.0, size=(S, 1, 2, 64, d)).astype(np.float32)
    lp = rng.normal(0.0, 3.0, size=(S, 1, 2, 64)).astype(np.float32)
    om, lm = gpu_lib.lse_merge(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda(), dtype=torch.float16)
    torch.cuda.synchronize()
    rom, rlm = oracle.ref_lse_merge(op.astype(np.float64), lp.astype(np.float64))
    assert om.dtype == torch.float16
    assert np.abs(_np(om) - rom).max() <= 2.0 ** -10 * np.abs(rom).max() + 1e-5
    assert np.abs(_np(lm) - rlm).max() <= 1e-5 + 1e-6 * np.abs(rlm).max()
