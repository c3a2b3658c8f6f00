"""The library's calls under HIP graph capture and on concurrent streams.

The entry points only validate their arguments and launch kernels on the
caller's stream (no allocation, no memset, no synchronisation), so a captured
graph must reproduce the eager results bit for bit on every replay, and calls
on two streams at once must give the same bits as the same calls made one
after the other.  Replays are interleaved with eager work on the same buffers
and with synchronisations, and every replay is checked.
"""
from __future__ import annotations

import pytest
import torch

from aware_exact_attention_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


def _inputs(seed, N=1000, H=4, d=128, dtype="bf16"):
    return [t.cuda() for t in make_inputs(1, H, N, d, dtype, seed=seed, backward=True)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_graph_replays_match_eager(gpu_lib, dtype):
    fa = gpu_lib
    q, k, v, do = _inputs(2000, dtype=dtype)
    B, H, N, d = q.shape
    o, lse = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    grads = tuple(torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    o2, lse2 = torch.empty_like(q), torch.empty_like(lse)
    wss = torch.empty(max(fa.splitkv_workspace_bytes(B, H, N, d, 3), 16), dtype=torch.uint8, device="cuda")
    ow, lw = torch.empty_like(q), torch.empty_like(lse)

    def step():
        fa.fwd(q, k, v, causal=True, out=o, lse=lse)
        fa.bwd(q, k, v, o, lse, do, causal=True, workspace=ws, out=grads)
        fa.fwd_splitkv(q, k, v, causal=True, num_splits=3, workspace=wss, out=o2, lse=lse2)
        fa.fwd_window(q, k, v, 100, 20, out=ow, lse=lw)

    outs = (o, lse, *grads, o2, lse2, ow, lw)
    step()  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        # new inputs written in place, eager reference on them, then the replay
        fresh = _inputs(2100 + r, dtype=dtype)
        for dst, src in zip((q, k, v, do), fresh):
            dst.copy_(src)
        step()
        torch.cuda.synchronize()
        want = [t.clone() for t in outs]
        for t in outs:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outs, want)):
            assert torch.equal(got, ref), f"replay {r}: output {i} differs from the eager result"


def test_two_streams_match_sequential(gpu_lib):
    fa = gpu_lib
    sets = [_inputs(2200), _inputs(2201, N=777, H=3)]
    seq = []
    for q, k, v, do in sets:
        o, lse = fa.fwd(q, k, v, causal=False)
        seq.append((o, lse, *fa.bwd(q, k, v, o, lse, do, causal=False)))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    cur = torch.cuda.current_stream()
    for s in streams:
        s.wait_stream(cur)
    par = [None, None]
    for rep in range(3):
        for i, ((q, k, v, do), s) in enumerate(zip(sets, streams)):
            with torch.cuda.stream(s):
                o, lse = fa.fwd(q, k, v, causal=False)
                par[i] = (o, lse, *fa.bwd(q, k, v, o, lse, do, causal=False))
        torch.cuda.synchronize()
        for i in range(2):
            for a, b in zip(par[i], seq[i]):
                assert torch.equal(a, b), f"stream {i}, repetition {rep}: differs from the sequential result"
