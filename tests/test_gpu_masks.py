"""GPU parity of the sliding-window and block-sparse forwards (through the C ABI).

Both have the contract of ``fa_fwd`` with a different visible set, so they are
held to the same tolerances against the fp64 oracle of ``oracle/masks.py``
(O max-abs 2e-2 / mean-abs 2e-3, LSE 1e-3).  Rows that see no key (possible
only under a block mask) must come back as exactly O = 0 and LSE = -inf.
Small sizes are compared in full; the full-size cases (N = 16384, the window
of the pages' SDPA example, and a half-dense block mask) on sampled rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from aware_exact_attention_amd.inputs import make_inputs, to_f64
from test_gpu_parity import _gpu, _np, _report, check_lse, check_o, sample_rows

pytestmark = pytest.mark.gpu

WINDOWS = [(-1, -1), (-1, 0), (0, 0), (5, 3), (100, 0), (63, 64), (512, 512), (0, -1)]


def _nan_outputs(q):
    B, H, N, d = q.shape
    return (torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device="cuda"),
            torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("N", [1, 100, 1000, 3000])
@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("window", WINDOWS, ids=[f"{a}_{b}" for a, b in WINDOWS])
def test_window_small(gpu_lib, N, d, window):
    left, right = window
    q, k, v = make_inputs(1, 2, N, d, "bf16", seed=800 + N + d)
    scale = d ** -0.5
    qd, kd, vd = _gpu(q, k, v)
    o, lse = _nan_outputs(qd)
    gpu_lib.fwd_window(qd, kd, vd, left, right, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.ref_fwd_window(to_f64(q), to_f64(k), to_f64(v), scale, left, right)
    tag = f"window N={N} d={d} ({left},{right})"
    check_o(tag, _np(o), ro)
    check_lse(tag, _np(lse), rl)


def _random_block_mask(H, nb, density, seed, per_head, empty_rows=True):
    rng = np.random.default_rng(seed)
    shape = (H, nb, nb) if per_head else (nb, nb)
    m = (rng.random(shape) < density).astype(np.uint8)
    if empty_rows and nb > 1:
        if per_head:
            m[0, 1] = 0          # head 0: block row 1 sees no key
        else:
            m[nb - 1] = 0        # last block row sees no key
    return m


def _check_blocksparse(tag, o, lse, ro, rl):
    empty = np.isinf(rl)
    assert np.array_equal(np.isinf(lse), empty), f"{tag}: rows without keys differ"
    assert np.all(lse[empty] == -np.inf) and np.all(o[empty] == 0), f"{tag}: empty rows not O=0, LSE=-inf"
    full = ~empty
    if full.any():
        check_o(tag, o[full], ro[full])
        check_lse(tag, lse[full], rl[full])


@pytest.mark.parametrize("N", [64, 130, 1000, 2049])
@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("per_head", [False, True])
def test_blocksparse_small(gpu_lib, N, d, causal, per_head):
    H = 3
    q, k, v = make_inputs(1, H, N, d, "bf16", seed=900 + N + d)
    scale = d ** -0.5
    nb = (N + 63) // 64
    bm = _random_block_mask(H, nb, 0.5, N + d + int(causal), per_head)
    qd, kd, vd = _gpu(q, k, v)
    o, lse = _nan_outputs(qd)
    gpu_lib.fwd_blocksparse(qd, kd, vd, torch.from_numpy(bm).cuda(), causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.ref_fwd_blocksparse(to_f64(q), to_f64(k), to_f64(v), scale, causal, bm)
    _check_blocksparse(f"blocksparse N={N} d={d} causal={causal} per_head={per_head}", _np(o), _np(lse), ro, rl)


def test_blocksparse_all_ones_equals_dense(gpu_lib):
    # a grid that fills the GPU, where the dense forward gives each row to one
    # wave (on small grids it splits a row's keys over several waves)
    q, k, v = _gpu(*make_inputs(4, 16, 1000, 128, "bf16", seed=950))
    nb = (1000 + 63) // 64
    for causal in (False, True):
        o1, l1 = gpu_lib.fwd(q, k, v, causal=causal)
        o2, l2 = gpu_lib.fwd_blocksparse(q, k, v, torch.ones((nb, nb), dtype=torch.uint8, device="cuda"),
                                         causal=causal)
        torch.cuda.synchronize()
        # the same tiles in the same order through the same kernel code: identical results
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("case", ["window_512", "blocks_half", "blocks_causal_heads"])
def test_masks_full_size_sampled(gpu_lib, case):
    if case == "window_512":
        B, H, N, d, causal = 1, 8, 16384, 128, False
    elif case == "blocks_half":
        B, H, N, d, causal = 1, 8, 16384, 128, False
    else:
        B, H, N, d, causal = 2, 4, 8192, 128, True
    q, k, v = make_inputs(B, H, N, d, "bf16", seed=960 + len(case))
    scale = d ** -0.5
    qd, kd, vd = _gpu(q, k, v)
    nb = (N + 63) // 64
    if case == "window_512":
        o, lse = gpu_lib.fwd_window(qd, kd, vd, 512, 512, scale=scale)
        bm = None
    else:
        per_head = case == "blocks_causal_heads"
        bm = _random_block_mask(H, nb, 0.5, 970, per_head)
        o, lse = gpu_lib.fwd_blocksparse(qd, kd, vd, torch.from_numpy(bm).cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = _np(o), _np(lse)
    qn, kn, vn = to_f64(q), to_f64(k), to_f64(v)
    rng = np.random.default_rng(N)
    for b in range(B):
        for h in range(H):
            rows = sample_rows(N, rng, extra=96)
            if bm is None:
                ro, rl = oracle.ref_fwd_window_rows(qn[b, h], kn[b, h], vn[b, h], scale, 512, 512, rows)
            else:
                mh = bm[h] if bm.ndim == 3 else bm
                ro, rl = oracle.ref_fwd_blocksparse_rows(qn[b, h], kn[b, h], vn[b, h], scale, causal, mh, rows)
            _check_blocksparse(f"{case} head=({b},{h})", o[b, h, rows], lse[b, h, rows], ro, rl)
