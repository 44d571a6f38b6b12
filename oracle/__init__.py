"""Oracle: a plain, slow, obviously correct CPU implementation of the
tile-signaled GEMM paths, used only as test infrastructure.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import anything from here.  The device library never calls it, shares
no code with it and must fail loudly when its own native code is missing.

Arithmetic is float64 over the exact values of the bf16 inputs; where the
method itself rounds an intermediate to bf16 (the activation fed to the second
GEMM), the oracle rounds the float64 value once, to nearest-even.  A numpy
float64 matrix product serves as the GEMM step; nothing is blocked, fused or
reordered beyond the definitions cited in each function.

Page citations:
  [TL]  "TileLink: Generating Efficient Compute-Communication Overlapping
        Kernels using Tile-Centric Primitives" (arXiv 2503.20313).
  [TD]  "Triton-distributed: Programming Overlapping Kernels on Distributed AI
        Systems with the Triton Compiler" (arXiv 2504.19442).
  [DG]  Digest page "Resource-aware Computation-Communication Overlap for
        multi-GPU ML Workloads": the CTA-pipelining abstract and the abstract on
        MoE expert compute overlapped with the return all-to-all through
        tile-level signaling.

Every function here is pinned by CPU tests (tests/test_oracle_*.py) against
brute force, closed forms, library routines or invariants; none is
"parity unpinned".
"""
from .numerics import bf16_to_f64, f64_to_bf16_bits, gelu_erf, silu  # noqa: F401
from .paths import (  # noqa: F401
    static_map_ag,
    ag_gather,
    gemm,
    gemm_abs,
    ag_gemm,
    rs_reduce,
    gemm_rs,
    mlp2,
    moe_route,
    moe_tile_table,
    moe_expert_combine,
    moe_ag_up,
    attention,
    ag_kv_attention,
    overlap_ratio,
)
