"""isk_attn_decode_static (the library's fixed device workspace) against
isk_attn_decode with a workspace of the caller's, through the C ABI.

Same kernels, so the same bits: two calls in a row, the second with a
smaller batch (the array keeps the first call's contents), on dense and
sparse 128-head batches with the split list in the kernel arguments, a
sparse batch of more than 128 rows (split list uploaded) and a dense 64-head
batch; a plan that needs more than the array holds is refused before
anything runs.
"""

import math

import numpy as np
import pytest
import torch

import invariant_split_kv_amd as isk
from workloads import synth
from workloads.device import DeviceCase

pytestmark = pytest.mark.gpu


def both(case):
    """(bits via a workspace of its own, bits via the static workspace)."""
    dc = DeviceCase(case)
    dc.run()
    _, _, bits, lbits = dc.result()
    out = torch.full_like(dc.out, float("nan"))
    lse = torch.full_like(dc.lse, float("nan"))
    isk.attn_decode_static(dc.plan.handle, dc.q, dc.pool, dc.block_table, dc.lens, dc.topk_idx, dc.topk_len,
                           out, lse)
    torch.cuda.synchronize()
    sbits = out.view(torch.int16).cpu().numpy()
    slbits = lse.view(torch.int32).cpu().numpy()
    dc.close()
    return (bits, lbits), (sbits, slbits)


@pytest.mark.parametrize("kind", ["dense_h128", "sparse_h128", "sparse_h128_uploaded", "dense_h64"])
def test_static_workspace_matches_own_workspace(kind):
    rng = np.random.default_rng(120)
    for step, B in enumerate((140, 130) if kind == "sparse_h128_uploaded" else (24, 5)):   # the second is smaller
        lens = rng.integers(1, 6000, B)
        if kind.startswith("sparse_h128"):
            case = synth.mla_case(lens, 128, 1.0 / math.sqrt(192.0), 64, structure_seed=121 + step, topk_width=1024)
        else:
            case = synth.mla_case(lens, 128 if kind == "dense_h128" else 64, 1.0 / math.sqrt(192.0), 64,
                                  structure_seed=121 + step)
        print(f"[case] static workspace {kind} call {step}: B={B}", flush=True)
        own, static = both(case)
        assert np.array_equal(own[0], static[0]) and np.array_equal(own[1], static[1]), \
            f"{kind} call {step}: static-workspace bits differ"


def test_static_workspace_refuses_a_plan_larger_than_it():
    # 64 rows of 20000 tokens, fp32 output, 64-token splits: ~20000 partials
    desc = isk.IskDesc(isk.KIND_MLA, 128, 1, synth.MLA_DQK, synth.MLA_DV, 64, 64 * 320, 320, 0, isk.SPLIT_PER_ROW,
                       64, isk.OUT_F32, 0, 0.07)
    with isk.Plan(desc, np.full(64, 20000, np.int32)) as plan:
        assert plan.workspace_bytes > (64 << 20)
        with pytest.raises(isk.IskError) as e:
            isk.attn_decode_static(plan.handle, None, None, None, None, None, None, None, None)
        assert e.value.status == -3 and "static workspace" in e.value.message
