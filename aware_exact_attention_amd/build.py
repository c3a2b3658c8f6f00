"""Build libfa.so (gfx950 only) in-tree with hipcc.

Usage: ``python -m aware_exact_attention_amd.build`` (or ``build()`` from Python).
Every call recompiles.  The library lands next to this file as ``libfa.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-munsafe-fp-atomics",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the backward's per-step S and dP accumulators feed
    # VALU work directly, and with the AGPR form the register allocator parks
    # the long-lived dK/dV accumulators in VGPRs and copies them back and
    # forth every step (the forward kernels are unaffected)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-result",
]


def build(verbose: bool = False, extra_flags=None) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), "-I", os.path.join(HERE, "..", "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
