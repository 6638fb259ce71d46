"""Shared helpers of the GPU tests: oracle references for synthetic cases and
the parity bar.

Parity bar (bf16 output): every element satisfies
    |gpu - ref| <= max(2e-3, ulp_bf16(ref))
where ulp_bf16(x) is the spacing of bf16 numbers at |x|.  Rounding the exact
result to bf16 alone can move it by half a ulp, which exceeds 2e-3 once
|ref| >= 0.5, so the bar allows one bf16 ulp of the exact value there and is
exactly 2e-3 below.  fp32 output: |gpu - ref| <= 2e-3 everywhere.  LSE
(natural log of the scaled scores): |gpu - ref| <= 1e-3; -inf must match.
"""

from __future__ import annotations

import sys

import numpy as np

import oracle
from workloads import synth

OUT_ATOL = 2e-3
LSE_ATOL = 1e-3


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def reference(case):
    """Oracle (out, lse) in float64 for a synthetic case."""
    q = synth.bf16_value(case.q_bits())
    if isinstance(case, synth.GqaCase):
        ks = [synth.bf16_value(r.k) for r in case.rows]
        vs = [synth.bf16_value(r.v) for r in case.rows]
        return oracle.gqa_decode(q, ks, vs, case.scale)
    if case.sparse and case.extra is not None:
        x = case.extra
        return oracle.mla_sparse_extra_decode(q, list(case.logical_rows()), case.lens, case.topk_idx(),
                                              case.topk_len(), list(x.logical_rows()), x.lens, x.topk_idx(),
                                              x.topk_len(), case.scale, dv=synth.MLA_DV)
    if case.sparse:
        return oracle.mla_sparse_decode(q, list(case.logical_rows()), case.lens, case.topk_idx(),
                                        case.topk_len(), case.scale, dv=synth.MLA_DV)
    return oracle.mla_decode(q, list(case.logical_rows()), case.scale, dv=synth.MLA_DV)


def parity(out, lse, ref_out, ref_lse, out_f32=False, what=""):
    """Assert the parity bar; returns a small report dict."""
    out = np.asarray(out, np.float64)
    err = np.abs(out - ref_out)
    tol = np.full_like(ref_out, OUT_ATOL) if out_f32 else np.maximum(OUT_ATOL, bf16_ulp(ref_out))
    bad = err > tol
    lse_inf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), lse_inf), f"{what}: -inf pattern of lse differs"
    lerr = np.where(lse_inf, 0.0, np.abs(np.where(lse_inf, 0.0, lse) - np.where(lse_inf, 0.0, ref_lse)))
    rep = {
        "max_abs": float(err.max(initial=0.0)),
        "relaxed_elems": int(np.sum(err > OUT_ATOL)),
        "fail_elems": int(bad.sum()),
        "lse_max_abs": float(lerr.max(initial=0.0)),
        "elems": int(err.size),
    }
    print(f"[parity] {what}: {rep}", flush=True)
    sys.stdout.flush()
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside the bar; worst {rep}"
    assert rep["lse_max_abs"] <= LSE_ATOL, f"{what}: lse error {rep['lse_max_abs']}"
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    return rep
