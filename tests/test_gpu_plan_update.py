"""Uploaded plans re-planned with isk_plan_update as the batch grows.

A plan whose split list is uploaded (batches of more than 128 rows) gets its
pinned staging ring when it is made and re-sizes it in isk_plan_update when
the split list outgrows it; smaller per-row batches go to the kernels by
value; isk_attn_decode itself allocates nothing.  One plan is re-planned
through batches of growing size (and back down, crossing between the two
forms), each decoded and checked against the oracle, with the previous
step's decode still in flight when the next update runs.
"""

import math

import numpy as np
import pytest
import torch

import invariant_split_kv_amd as isk
from workloads import synth
from workloads.device import device_pool, _u16_to_bf16

from gpu_util import parity, reference

pytestmark = pytest.mark.gpu


def staged(case, max_pages):
    """Device inputs of a case, block table padded to `max_pages` columns."""
    bt = np.full((case.batch, max_pages), -1, np.int32)
    bt[:, :case.paging.max_pages_per_row] = case.paging.block_table
    d = dict(q=_u16_to_bf16(case.q_bits(), "cuda"), pool=device_pool(case),
             bt=torch.from_numpy(bt).cuda(), lens=torch.from_numpy(np.asarray(case.lens, np.int32)).cuda())
    if case.sparse:
        d["idx"] = torch.from_numpy(case.topk_idx()).cuda()
        d["tl"] = torch.from_numpy(case.topk_len()).cuda()
    return d


def check(out, lse, case, what):
    torch.cuda.synchronize()
    ro, rl = reference(case)
    parity(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, False, what)


@pytest.mark.parametrize("kind", ["sparse", "dense_over_128_rows"])
def test_uploaded_plan_across_update_growth(kind):
    rng = np.random.default_rng(90)
    sizes = [3, 40, 150, 260, 20] if kind == "sparse" else [130, 200, 320, 140]
    cases = []
    for i, B in enumerate(sizes):
        lens = rng.integers(1, 600, B)
        if kind == "sparse":
            cases.append(synth.mla_case(lens, 128, 0.08, 64, structure_seed=91 + i, topk_width=128))
        else:
            cases.append(synth.mla_case(lens, 128, 0.08, 64, structure_seed=91 + i))
    num_pages = max(c.paging.num_pages for c in cases)
    max_pages = max(c.paging.max_pages_per_row for c in cases)
    c0 = cases[0]
    desc = isk.IskDesc(isk.KIND_MLA, 128, 1, synth.MLA_DQK, synth.MLA_DV, 64, num_pages, max_pages,
                       c0.topk_width, isk.SPLIT_PER_ROW, 0, isk.OUT_BF16, 0, c0.scale)
    stream = torch.cuda.current_stream()
    plan = isk.Plan(desc, np.asarray(c0.lens, np.int32), c0.topk_len() if kind == "sparse" else None)
    prev = None
    try:
        for i, case in enumerate(cases):
            if i > 0:   # the previous step's decode is still in flight here
                plan.update(np.asarray(case.lens, np.int32), case.topk_len() if kind == "sparse" else None)
            info = plan.info()
            print(f"[case] {kind} step {i}: B={case.batch} splits={info['num_segments']} "
                  f"workspace={plan.workspace_bytes}", flush=True)
            d = staged(case, max_pages)
            ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
            out = torch.empty((case.batch, 128, synth.MLA_DV), dtype=torch.bfloat16, device="cuda")
            lse = torch.empty((case.batch, 128), dtype=torch.float32, device="cuda")
            isk.attn_decode(plan.handle, d["q"], d["pool"], d["bt"], d["lens"], d.get("idx"), d.get("tl"), out,
                            lse, ws, ws.numel(), stream)
            if prev is not None:
                check(*prev)
            prev = (out, lse, case, f"{kind} step {i} B={case.batch}")
            del d, ws
        check(*prev)
    finally:
        plan.close()


def test_threads_decode_with_one_uploaded_plan():
    """Four host threads decode with one uploaded (sparse, 140 rows) plan at
    the same time, each on its own stream with its own workspace and outputs:
    the plan's staging ring hands each call its own slot, and every output
    has the bits of a single-threaded decode."""
    import threading
    case = synth.mla_case(np.random.default_rng(95).integers(100, 3000, 140), 128, 0.08, 64, structure_seed=96,
                          topk_width=512)
    desc = isk.IskDesc(isk.KIND_MLA, 128, 1, synth.MLA_DQK, synth.MLA_DV, 64, case.paging.num_pages,
                       case.paging.max_pages_per_row, case.topk_width, isk.SPLIT_PER_ROW, 0, isk.OUT_BF16, 0,
                       case.scale)
    d = staged(case, case.paging.max_pages_per_row)
    plan = isk.Plan(desc, np.asarray(case.lens, np.int32), case.topk_len())
    try:
        def one(stream):
            ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
            out = torch.empty((case.batch, 128, synth.MLA_DV), dtype=torch.bfloat16, device="cuda")
            lse = torch.empty((case.batch, 128), dtype=torch.float32, device="cuda")
            isk.attn_decode(plan.handle, d["q"], d["pool"], d["bt"], d["lens"], d["idx"], d["tl"], out, lse, ws,
                            ws.numel(), stream)
            return out, lse, ws
        ref_out, ref_lse, _ = one(torch.cuda.current_stream())
        torch.cuda.synchronize()
        ref = (ref_out.view(torch.int16).cpu().numpy(), ref_lse.view(torch.int32).cpu().numpy())
        results, errors = [], []

        def worker(k):
            try:
                s = torch.cuda.Stream()
                mine = [one(s) for _ in range(20)]
                s.synchronize()
                results.extend((o.view(torch.int16).cpu().numpy(), l.view(torch.int32).cpu().numpy())
                               for o, l, _ in mine)
            except Exception as e:   # surfaced below
                errors.append(repr(e))

        threads = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        assert not errors, errors
        assert len(results) == 80
        for o, l in results:
            assert np.array_equal(o, ref[0]) and np.array_equal(l, ref[1])
    finally:
        torch.cuda.synchronize()
        plan.close()
