"""CPU oracle for batch-invariant split-KV decode attention (fp64, numpy).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path never imports it.
"""
from .attention import (attend, gqa_decode, merge, merge_many, mla_decode,
                        mla_sparse_decode, mla_sparse_extra_decode, sparse_positions)
from .gemm import linear
from .norm import rmsnorm

__all__ = ["attend", "gqa_decode", "mla_decode", "mla_sparse_decode",
           "mla_sparse_extra_decode", "sparse_positions", "merge", "merge_many", "rmsnorm", "linear"]
