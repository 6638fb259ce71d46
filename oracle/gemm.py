"""Oracle for the batch-invariant matmul: plain, fp64, CPU.

TEST INFRASTRUCTURE ONLY.  Only the test suite and the benchmark's
CPU-baseline leg may import this module; it shares no code with the HIP path.

The gllm issue "Greedy outputs depend on batch composition (NVFP4 GEMV/GEMM
switch at 32 rows is a candidate)" (sections "Candidate cause" and "Next
steps") traces batch dependence to a kernel switch by row count whose two
sides round the activations differently, and proposes that both sides use
the same activation precision so the switch changes speed, not results.
What either side computes is the plain product of the given operands:

    y[m, n] = sum_k x[m, k] * w[n, k]

evaluated here in float64 on the exact (bf16) input values.
"""

from __future__ import annotations

import numpy as np

__all__ = ["linear"]


def linear(x, w):
    """x: [M, K]; w: [N, K] (one row per output feature); returns [M, N]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T
