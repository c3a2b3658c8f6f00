"""GPU parity of the sliding-window and block-sparse backward (through the C ABI).

The gradients are held to the dense backward's tolerances (max-abs 2e-2 and
mean-abs 1e-2 relative to the fp64 oracle's largest and mean magnitude) against
``oracle.ref_bwd_window`` / ``oracle.ref_bwd_blocksparse``, with o and lse from
the library's own masked forward.  Rows that see no key must come back with dq
rows of exactly 0.  Small and ragged sizes are compared in full, and so is a
4096-row case of the pages' (512, 512) window and of a half-dense block mask.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from aware_exact_attention_amd.inputs import make_inputs, to_f64
from test_gpu_masks import _random_block_mask
from test_gpu_parity import ZERO_REF_ATOL, _gpu, _np, check_grad

pytestmark = pytest.mark.gpu

WINDOWS = [(-1, -1), (-1, 0), (0, 0), (5, 3), (100, 0), (63, 64), (0, -1), (200, 10)]


def _nan3(q):
    return tuple(torch.full_like(q, float("nan")) for _ in range(3))


# Gradients that are exactly 0 in exact arithmetic (window (0, 0)) are held to
# ZERO_REF_ATOL, derived where check_grad is defined.


def _check3(tag, got, ref):
    for what, g, r in zip(("dQ", "dK", "dV"), got, ref):
        if not np.abs(r).max() > 0:
            err = float(np.abs(g - r).max())
            assert np.isfinite(g).all() and err <= ZERO_REF_ATOL, f"{tag}: {what} max-abs {err:.3e} (ref is 0)"
            continue
        check_grad(tag, what, g, r)


def _window_case(fa, q, k, v, do, left, right, scale):
    qd, kd, vd, dod = _gpu(q, k, v, do)
    o, lse = fa.fwd_window(qd, kd, vd, left, right, scale=scale)
    g = fa.bwd_window(qd, kd, vd, o, lse, dod, left, right, scale=scale, out=_nan3(qd))
    torch.cuda.synchronize()
    return tuple(_np(t) for t in g)


@pytest.mark.parametrize("N", [1, 100, 300, 1000])
@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("window", WINDOWS, ids=[f"{a}_{b}" for a, b in WINDOWS])
def test_window_bwd_small(gpu_lib, N, d, window):
    left, right = window
    q, k, v, do = make_inputs(1, 2, N, d, "bf16", seed=1100 + N + d, backward=True)
    scale = d ** -0.5
    got = _window_case(gpu_lib, q, k, v, do, left, right, scale)
    ref = oracle.ref_bwd_window(*(to_f64(t) for t in (q, k, v, do)), scale, left, right)
    _check3(f"bwd window N={N} d={d} ({left},{right})", got, ref)


def _blocks_case(fa, q, k, v, do, bm, causal, scale):
    qd, kd, vd, dod = _gpu(q, k, v, do)
    m = torch.from_numpy(bm).cuda()
    o, lse = fa.fwd_blocksparse(qd, kd, vd, m, causal=causal, scale=scale)
    g = fa.bwd_blocksparse(qd, kd, vd, o, lse, dod, m, causal=causal, scale=scale, out=_nan3(qd))
    torch.cuda.synchronize()
    return tuple(_np(t) for t in g)


def _check_blocks(tag, got, ref, bm, causal, N):
    H = got[0].shape[1]
    for h in range(H):
        mh = bm[h] if bm.ndim == 3 else bm
        vis = np.repeat(np.repeat(mh != 0, 64, 0), 64, 1)[:N, :N]
        if causal:
            vis &= np.tril(np.ones((N, N), dtype=bool))
        empty = ~vis.any(axis=1)
        assert np.all(got[0][:, h][:, empty] == 0), f"{tag}: dq of rows without keys is not 0 (head {h})"
    _check3(tag, got, ref)


@pytest.mark.parametrize("N", [64, 130, 1000])
@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("per_head", [False, True])
def test_blocksparse_bwd_small(gpu_lib, N, d, causal, per_head):
    H = 3
    q, k, v, do = make_inputs(1, H, N, d, "bf16", seed=1200 + N + d, backward=True)
    scale = d ** -0.5
    nb = (N + 63) // 64
    bm = _random_block_mask(H, nb, 0.5, N + d + int(causal) + 7, per_head)
    got = _blocks_case(gpu_lib, q, k, v, do, bm, causal, scale)
    ref = oracle.ref_bwd_blocksparse(*(to_f64(t) for t in (q, k, v, do)), scale, causal, bm)
    _check_blocks(f"bwd blocksparse N={N} d={d} causal={causal} per_head={per_head}", got, ref, bm, causal, N)


@pytest.mark.parametrize("H,N", [(2, 300), (128, 200)])
@pytest.mark.parametrize("d", [64, 96, 128, 256])
def test_masks_bwd_each_launch_shape(gpu_lib, H, N, d):
    """The mask backwards run their two passes in one grid when both fit on
    the 256 CUs together (B1 H2 N300) and as two launches otherwise (B1 H128
    N200: 256 + 256 workgroups at d = 128).  Window (5, 3) and a random
    per-head block mask with the causal limit, compared in full."""
    q, k, v, do = make_inputs(1, H, N, d, "bf16", seed=1700 + H + N + d, backward=True)
    scale = d ** -0.5
    args64 = [to_f64(t) for t in (q, k, v, do)]
    got = _window_case(gpu_lib, q, k, v, do, 5, 3, scale)
    _check3(f"bwd window launch shape H={H} N={N} d={d}", got, oracle.ref_bwd_window(*args64, scale, 5, 3))
    bm = _random_block_mask(H, (N + 63) // 64, 0.5, 1710 + H + N + d, True)
    got = _blocks_case(gpu_lib, q, k, v, do, bm, True, scale)
    ref = oracle.ref_bwd_blocksparse(*args64, scale, True, bm)
    _check_blocks(f"bwd blocksparse launch shape H={H} N={N} d={d}", got, ref, bm, True, N)


@pytest.mark.parametrize("d", [64, 128])
def test_window_bwd_persistent(gpu_lib, d):
    """Window (40, 70) over B2 H96 N300: 576 key blocks, so the dK/dV pass runs
    as persistent workgroups that bring each block's K, V and first tiles in
    during the previous block; the blocks' query-step ranges differ at both
    ends.  Compared in full."""
    q, k, v, do = make_inputs(2, 96, 300, d, "bf16", seed=1760 + d, backward=True)
    scale = d ** -0.5
    got = _window_case(gpu_lib, q, k, v, do, 40, 70, scale)
    _check3(f"bwd window persistent d={d}", got, oracle.ref_bwd_window(*(to_f64(t) for t in (q, k, v, do)),
                                                                       scale, 40, 70))


def test_blocksparse_bwd_all_ones_equals_dense(gpu_lib):
    """An all-ones mask visits the same steps and tiles in the same order as
    the dense backward, so the gradients agree bit for bit."""
    q, k, v, do = _gpu(*make_inputs(2, 4, 1000, 128, "bf16", seed=1250, backward=True))
    nb = (1000 + 63) // 64
    ones = torch.ones((nb, nb), dtype=torch.uint8, device="cuda")
    for causal in (False, True):
        o, lse = gpu_lib.fwd(q, k, v, causal=causal)
        a = gpu_lib.bwd(q, k, v, o, lse, do, causal=causal)
        b = gpu_lib.bwd_blocksparse(q, k, v, o, lse, do, ones, causal=causal)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y)


@pytest.mark.parametrize("case", ["window_512", "blocks_half", "blocks_causal_heads"])
def test_masks_bwd_4096(gpu_lib, case):
    B, H, N, d = 1, 2, 4096, 128
    causal = case == "blocks_causal_heads"
    q, k, v, do = make_inputs(B, H, N, d, "bf16", seed=1300 + len(case), backward=True)
    scale = d ** -0.5
    args64 = [to_f64(t) for t in (q, k, v, do)]
    if case == "window_512":
        got = _window_case(gpu_lib, q, k, v, do, 512, 512, scale)
        _check3(case, got, oracle.ref_bwd_window(*args64, scale, 512, 512))
    else:
        bm = _random_block_mask(H, N // 64, 0.5, 1310, per_head=causal)
        got = _blocks_case(gpu_lib, q, k, v, do, bm, causal, scale)
        _check_blocks(case, got, oracle.ref_bwd_blocksparse(*args64, scale, causal, bm), bm, causal, N)
