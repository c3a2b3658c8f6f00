"""Exact tiled attention for MI355X (gfx950): HIP kernels behind a C ABI (libfa.so).

``aware_exact_attention_amd.fa`` is the Python binding (``fwd``, ``bwd``);
``aware_exact_attention_amd.inputs`` holds the seeded synthetic workloads;
``aware_exact_attention_amd.build`` compiles the library in-tree.
"""
