"""Oracle for batch-invariant RMSNorm: plain, slow, fp64, CPU.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; it shares no code with
the HIP path.

The inference-research gotcha "batch-invariance-is-not-universal-across-
kernel-paths" (section "Root cause") names small-batch split reductions in
RMSNorm among the strategies that make a kernel's output depend on the batch.
The pages do not restate the operation; the reading taken here is the usual
definition of RMS normalisation with a per-channel weight:

    y[r, i] = x[r, i] / sqrt(mean_j x[r, j]^2 + eps) * w[i]

computed on the given input values in float64.
"""

from __future__ import annotations

import numpy as np

__all__ = ["rmsnorm"]


def rmsnorm(x, w, eps: float):
    """x: [rows, dim]; w: [dim]; returns y [rows, dim] (float64)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    ms = np.mean(x * x, axis=1, keepdims=True)      # mean of squares per row
    return x / np.sqrt(ms + float(eps)) * w[None, :]
