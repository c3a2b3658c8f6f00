"""Seeded synthetic inputs and the named workloads.

This module holds no attention arithmetic: it only draws i.i.d. normal
tensors with a fixed seed and rounds them once to the storage dtype.  Both the
HIP path (after a copy to the device) and the CPU oracle (after widening to
float64) read exactly these values.

Recipe: ``torch.Generator().manual_seed(seed)``, then ``torch.randn`` in
float32 on the CPU for Q, K, V and, for backward workloads, dO, in that order.
``qk_std`` multiplies Q and K in float32 before the single round-to-nearest-even
conversion to bfloat16 (or float16 for ``dtype="fp16"``; float32 workloads are
not rounded).

The shapes follow the pages' workloads: the benchmark harness of the
FlashAttention-2 principle and deployment page (B=1, H=8, d=128, bf16 randn,
N from 2K to 16K) and the GPT-2 shape (N=1024, d=64) quoted in the Journal of
Software 2026(1) p.218 survey.  No dataset is involved.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "bf16", "fp16" or "f32"
    causal: bool
    seed: int
    qk_std: float = 1.0
    backward: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def fwd_flop(self) -> float:
        """4*B*H*N^2*d, halved for causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    @property
    def bwd_flop(self) -> float:
        """10*B*H*N^2*d (five N x N x d products, one of them the recompute), halved for causal."""
        f = 10.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 256, 64, "f32", False, 0),
    "gpt2": Workload("gpt2", 8, 12, 1024, 64, "bf16", False, 1),
    "gpt2_causal": Workload("gpt2_causal", 8, 12, 1024, 64, "bf16", True, 1),
    "sweep_2k": Workload("sweep_2k", 1, 8, 2048, 128, "bf16", False, 2),
    "sweep_4k": Workload("sweep_4k", 1, 8, 4096, 128, "bf16", False, 2),
    "sweep_8k": Workload("sweep_8k", 1, 8, 8192, 128, "bf16", False, 2),
    "sweep_16k": Workload("sweep_16k", 1, 8, 16384, 128, "bf16", False, 2),
    "stress_causal": Workload("stress_causal", 2, 8, 16000, 128, "bf16", True, 3, qk_std=3.0),
    "fwd_bwd_causal": Workload("fwd_bwd_causal", 4, 16, 4096, 128, "bf16", True, 4, backward=True),
    "bwd_16k": Workload("bwd_16k", 1, 8, 16384, 128, "bf16", False, 5, backward=True),
}


def make_inputs(B: int, H: int, N: int, d: int, dtype: str = "bf16", seed: int = 0,
                qk_std: float = 1.0, backward: bool = False):
    """Return CPU tensors ``(q, k, v)`` or ``(q, k, v, do)``, each ``[B,H,N,d]`` contiguous."""
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, N, d)
    names = ["q", "k", "v"] + (["do"] if backward else [])
    out = []
    for name in names:
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if name in ("q", "k") and qk_std != 1.0:
            x = x * qk_std
        if dtype == "bf16":
            x = x.to(torch.bfloat16)
        elif dtype == "fp16":
            x = x.to(torch.float16)
        elif dtype != "f32":
            raise ValueError(f"unknown dtype {dtype!r}")
        out.append(x.contiguous())
    return tuple(out)


def workload_inputs(w: Workload):
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.qk_std, w.backward)


def to_f64(t: torch.Tensor):
    """Widen a CPU tensor to a float64 numpy array (exact for bf16, fp16 and fp32)."""
    return t.detach().to("cpu", torch.float64).numpy()
