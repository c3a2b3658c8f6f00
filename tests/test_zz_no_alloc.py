"""GPU check of fa_bwd_noalloc, the backward that takes no workspace and
allocates nothing: through the C ABI, its gradients against those of fa_bwd
(same kernels, so bit for bit) and against the fp64 oracle at the backward's
tolerances, on two calls in a row, the second with a smaller problem (the
library's scratch still holds the first call's row terms then)."""
from __future__ import annotations

import pytest
import torch

import oracle
from aware_exact_attention_amd.inputs import make_inputs, to_f64
from test_gpu_parity import _np, check_grad

pytestmark = pytest.mark.gpu

CASES = [(2, 8, 1000, 128, True, 2101), (1, 3, 300, 64, False, 2102)]


def _run(fa, B, H, N, d, causal, seed):
    q, k, v, do = make_inputs(B, H, N, d, "bf16", seed=seed, backward=True)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal=causal)
    ref = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal)
    out = tuple(torch.full_like(qd, float("nan")) for _ in range(3))
    got = fa.bwd_noalloc(qd, kd, vd, o, lse, dod, out, causal=causal)
    torch.cuda.synchronize()
    return (q, k, v, do), ref, got


def test_noalloc_matches_fa_bwd_twice(gpu_lib):
    for B, H, N, d, causal, seed in CASES:
        print(f"fa_bwd_noalloc B={B} H={H} N={N} d={d} causal={causal}", flush=True)
        ins, ref, got = _run(gpu_lib, B, H, N, d, causal, seed)
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.isfinite(a).all().item(), f"{name}: unwritten or non-finite"
            assert torch.equal(a, b), f"{name}: fa_bwd_noalloc differs from fa_bwd"
        rq, rk, rv = oracle.ref_bwd(*(to_f64(t) for t in ins), d ** -0.5, causal)
        tag = f"noalloc B={B} H={H} N={N} d={d} causal={causal}"
        for name, g, r in zip(("dQ", "dK", "dV"), got, (rq, rk, rv)):
            check_grad(tag, name, _np(g), r)


def test_noalloc_refuses_oversize(gpu_lib):
    """A problem whose workspace would not fit the 32 MiB scratch is refused
    before anything runs (validation only; the tensors are never read)."""
    B, H, N, d = 1, 1, (1 << 22) + 1, 64
    assert gpu_lib.bwd_workspace_bytes(B, H, N, d) > 32 << 20
    x = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    outs = tuple(torch.empty_like(x) for _ in range(3))
    with pytest.raises(gpu_lib.FAError) as e:
        gpu_lib.bwd_noalloc(x, x, x, x, lse, x, outs)
    assert e.value.status == -10
