"""Batch invariance of the HIP path: bit equality, not tolerance.

Protocols from the FlashMLA issue page "Sparse MLA decode is not
batch-invariant ..." (section "Measurement"): re-running identical inputs must
give identical bits (determinism control), and a row re-run alone with freshly
planned splits must give the bits it got inside the batch.  The differences
that page reports are 1-2 bf16 ulp, inside any tolerance, so every comparison
here is on raw output bits (bf16 out and fp32 lse).

The per-row split mode must pass every check; the batch-balanced comparison
mode is the negative control and must show at least one difference, which
proves the harness can see the effect.
"""

import math

import numpy as np
import pytest
import torch

import invariant_split_kv_amd as isk
from workloads import synth
from workloads.device import DeviceCase

from gpu_util import parity, reference

pytestmark = pytest.mark.gpu

MLA_SCALE = 1.0 / math.sqrt(192.0)


def run_bits(case, **kw):
    dc = DeviceCase(case, **kw)
    dc.run()
    r = dc.result()
    dc.close()
    return r


def solo_case(case, b, structure_seed):
    """Row b of `case` alone, in a freshly permuted page pool."""
    if isinstance(case, synth.GqaCase):
        one = synth.gqa_case([case.lens[b]], case.hq, case.hkv, case.d, case.scale, case.paging.page_size,
                             structure_seed, permute=True, split_tokens=case.split_tokens, seeds=[0])
        one.rows = [case.rows[b]]
        return one
    one = synth.mla_case([case.lens[b]], case.hq, case.scale, case.paging.page_size, structure_seed,
                         topk_width=case.topk_width, split_tokens=case.split_tokens, seeds=[0])
    one.rows = [case.rows[b]]
    if case.extra is not None:
        x = case.extra
        one.extra = synth.mla_case([x.lens[b]], case.hq, case.scale, x.paging.page_size, structure_seed + 1,
                                   topk_width=x.topk_width, split_tokens=case.split_tokens, seeds=[0])
        one.extra.rows = [x.rows[b]]
    return one


def test_repeat_runs_are_bit_identical():
    case = synth.config3_mla()
    dc = DeviceCase(case)
    first = None
    for i in range(10):
        dc.run()
        _, _, bits, lbits = dc.result()
        if first is None:
            first = (bits, lbits)
        else:
            assert np.array_equal(bits, first[0]) and np.array_equal(lbits, first[1]), f"run {i} differs"
    dc.close()


def test_cold_and_warm_cache_give_the_same_bits():
    case = synth.config3_mla(batch=16)
    dc = DeviceCase(case)
    dc.run()
    _, _, warm_b, warm_l = dc.result()
    dc.run()
    _, _, warm2_b, warm2_l = dc.result()
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    flush.fill_(1)
    torch.cuda.synchronize()
    dc.run()
    _, _, cold_b, cold_l = dc.result()
    dc.close()
    del flush
    assert np.array_equal(warm_b, cold_b) and np.array_equal(warm_l, cold_l)
    assert np.array_equal(warm_b, warm2_b)


GQA_GROUP_LENS = [1, 17, 64, 65, 500, 511, 512, 513, 1300, 2047, 3000, 4100]


def gqa_group_case(g, d):
    """GQA rows across split and tile edges with G query heads per kv head
    (the token-split kernel's G = 8 and 16 layouts)."""
    return synth.gqa_case(GQA_GROUP_LENS, 2 * g, 2, d, 1.0 / math.sqrt(d), 16, structure_seed=60 + g)


@pytest.mark.parametrize("which", ["config1", "config2", "config3", "config4", "config4_extra", "gqa_g8", "gqa_g16"])
def test_every_row_solo_equals_batched(which):
    case = {"config1": synth.config1_gqa_tiny, "config2": synth.config2_gqa,
            "config3": synth.config3_mla, "config4": synth.config4_sparse,
            "config4_extra": synth.config4_sparse_extra,
            "gqa_g8": lambda: gqa_group_case(8, 128), "gqa_g16": lambda: gqa_group_case(16, 64)}[which]()
    _, _, bits, lbits = run_bits(case)
    mism = []
    for b in range(case.batch):
        one = solo_case(case, b, structure_seed=1000 + b)
        _, _, sb, sl = run_bits(one)
        if not (np.array_equal(sb[0], bits[b]) and np.array_equal(sl[0], lbits[b])):
            mism.append(b)
    print(f"[invariance] {which}: {case.batch - len(mism)}/{case.batch} rows bit-identical solo vs batched", flush=True)
    assert not mism, f"{which}: rows {mism} differ between solo and batched runs"


def test_batch_permutation_keeps_row_bits():
    case = synth.config3_mla(batch=24)
    _, _, bits, lbits = run_bits(case)
    perm = np.random.default_rng(7).permutation(case.batch)
    pcase = synth.mla_case(case.lens[perm], case.hq, case.scale, 64, structure_seed=77, seeds=[0] * case.batch)
    pcase.rows = [case.rows[i] for i in perm]
    _, _, pbits, plbits = run_bits(pcase)
    assert np.array_equal(pbits, bits[perm]) and np.array_equal(plbits, lbits[perm])


# ------------------------------------------------------------ config-5 stress
#
# The probe row (len 16384, row seed 0) sits at a random position among
# batchmates with lengths uniform in [1, 131072].  Row content is generated on
# the GPU from each row's own seed (torch's seeded generator), so a row's
# values are the same in every batch that contains it.

def _gpu_row(seed, length, hq):
    g = torch.Generator(device="cuda")
    g.manual_seed(int(seed))
    q = (torch.randn((hq, synth.MLA_DQK), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    lat = (torch.randn((max(length, 1), synth.MLA_DQK), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    return q, lat[:length]


def _gpu_batch_run(lens, seeds, paging_seed, split_mode=isk.SPLIT_PER_ROW, hq=128, bands=None):
    lens = np.asarray(lens, dtype=np.int32)
    paging = synth.make_paging(lens, 64, np.random.default_rng(paging_seed))
    pool = torch.zeros((paging.num_pages * 64, synth.MLA_DQK), dtype=torch.bfloat16, device="cuda")
    qs = []
    for b, (L, s) in enumerate(zip(lens, seeds)):
        q, lat = _gpu_row(s, int(L), hq)
        qs.append(q)
        if L:
            pool[torch.from_numpy(paging.token_slots(b, np.arange(int(L)))).cuda()] = lat
    q = torch.stack(qs)
    desc = isk.IskDesc(isk.KIND_MLA, hq, 1, synth.MLA_DQK, synth.MLA_DV, 64, paging.num_pages,
                       paging.max_pages_per_row, 0, split_mode, 0, isk.OUT_BF16, 0, MLA_SCALE)
    bt = torch.from_numpy(paging.block_table).cuda()
    lens_d = torch.from_numpy(lens).cuda()
    out = torch.empty((len(lens), hq, synth.MLA_DV), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((len(lens), hq), dtype=torch.float32, device="cuda")
    with isk.Plan(desc, lens, bands=bands) as plan:
        ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
        isk.attn_decode(plan.handle, q, pool.view(paging.num_pages, 64, synth.MLA_DQK), bt, lens_d, None, None,
                        out, lse, ws, ws.numel())
        torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy(), lse.view(torch.int32).cpu().numpy(), q, pool, paging


_SOLO = {}


def _solo(seed, length, mode, bands=None):
    key = (seed, length, mode, None if bands is None else tuple(map(tuple, bands)))
    if key not in _SOLO:
        ob, lb, _, _, _ = _gpu_batch_run([length], [seed], paging_seed=9000 + len(_SOLO), split_mode=mode,
                                         bands=bands)
        _SOLO[key] = (ob[0], lb[0])
    return _SOLO[key]


@pytest.mark.parametrize("B", [1, 2, 8, 32, 128])
def test_config5_probe_bits_in_every_composition(B):
    probe = _solo(synth.PROBE_SEED, synth.PROBE_LEN, isk.SPLIT_PER_ROW)
    checked = 0
    for comp in range(3):
        lens, seeds, pos = synth.config5_composition(B, comp)
        print(f"[config5] B={B} composition={comp} probe at {pos} sum(len)={int(lens.sum())}", flush=True)
        ob, lb, _, _, _ = _gpu_batch_run(lens, seeds, paging_seed=100 * B + comp)
        assert np.array_equal(ob[pos], probe[0]) and np.array_equal(lb[pos], probe[1]), \
            f"probe differs at B={B} composition {comp}"
        others = [j for j in range(B) if j != pos]
        for j in np.random.default_rng([B, comp]).choice(others, size=min(8, len(others)), replace=False) if others else []:
            so = _solo(seeds[j], int(lens[j]), isk.SPLIT_PER_ROW)
            assert np.array_equal(ob[j], so[0]) and np.array_equal(lb[j], so[1]), \
                f"batchmate {j} (len {lens[j]}) differs from its solo run at B={B}"
            checked += 1
    print(f"[config5] B={B}: probe identical in 3/3 compositions, {checked} sampled batchmates identical", flush=True)


# A band table whose bands all touch the stress lengths: the probe (16384)
# takes the capped middle band, batchmates up to 131072 all three.
STRESS_BANDS = [(4096, 512), (20000, 1024, 10), (1 << 30, 2048, 24)]


@pytest.mark.parametrize("B", [2, 32, 128])
def test_config5_probe_bits_under_a_band_table(B):
    probe = _solo(synth.PROBE_SEED, synth.PROBE_LEN, isk.SPLIT_PER_ROW, STRESS_BANDS)
    for comp in range(2):
        lens, seeds, pos = synth.config5_composition(B, comp)
        print(f"[config5 bands] B={B} composition={comp} probe at {pos}", flush=True)
        ob, lb, _, _, _ = _gpu_batch_run(lens, seeds, paging_seed=100 * B + comp, bands=STRESS_BANDS)
        assert np.array_equal(ob[pos], probe[0]) and np.array_equal(lb[pos], probe[1]), \
            f"probe differs under the band table at B={B} composition {comp}"
        others = [j for j in range(B) if j != pos]
        for j in np.random.default_rng([B, comp, 1]).choice(others, size=min(4, len(others)), replace=False):
            so = _solo(seeds[j], int(lens[j]), isk.SPLIT_PER_ROW, STRESS_BANDS)
            assert np.array_equal(ob[j], so[0]) and np.array_equal(lb[j], so[1]), \
                f"batchmate {j} (len {lens[j]}) differs from its solo run under the band table at B={B}"


def test_config5_probe_matches_oracle():
    ob, lb, q, pool, paging = _gpu_batch_run([synth.PROBE_LEN], [synth.PROBE_SEED], paging_seed=4242)
    lat = pool[torch.from_numpy(paging.token_slots(0, np.arange(synth.PROBE_LEN))).cuda()]
    import oracle
    ro, rl = oracle.mla_decode(q.float().cpu().numpy(), [lat.float().cpu().numpy()], MLA_SCALE)
    out = torch.from_numpy(ob).view(torch.bfloat16).float().numpy()
    lse = torch.from_numpy(lb).view(torch.float32).numpy()
    parity(out, lse, ro, rl, False, "config5 probe")


def test_balanced_mode_is_caught_by_the_harness():
    """Negative control: the batch-wide balanced split changes probe bits."""
    solo = _solo(synth.PROBE_SEED, synth.PROBE_LEN, isk.SPLIT_BATCH_BALANCED)
    differing, total = 0, 0
    for B in (2, 8, 32, 128):
        for comp in range(3):
            lens, seeds, pos = synth.config5_composition(B, comp)
            ob, lb, _, _, _ = _gpu_batch_run(lens, seeds, paging_seed=7 * B + comp,
                                             split_mode=isk.SPLIT_BATCH_BALANCED)
            total += 1
            differing += int(not (np.array_equal(ob[pos], solo[0]) and np.array_equal(lb[pos], solo[1])))
    print(f"[negative control] balanced mode: probe bit-identical in {total - differing}/{total} compositions",
          flush=True)
    assert differing > 0


def test_config5_longest_batchmates_match_oracle():
    """The two longest batchmates of a B=32 stress composition (tens of
    thousands of tokens, more than 64 splits for the longest) against the
    oracle, so that an error shared by solo and batched runs (which the bit
    comparisons above cannot see) would still show."""
    lens, seeds, pos = synth.config5_composition(32, 0)
    ob, lb, q, pool, paging = _gpu_batch_run(lens, seeds, paging_seed=3200)
    import oracle
    longest = [int(j) for j in np.argsort(lens)[::-1][:2]]
    print(f"[config5 oracle] rows {longest} lens {[int(lens[j]) for j in longest]}", flush=True)
    for j in longest:
        L = int(lens[j])
        lat = pool[torch.from_numpy(paging.token_slots(j, np.arange(L))).cuda()]
        ro, rl = oracle.mla_decode(q[j:j + 1].float().cpu().numpy(), [lat.float().cpu().numpy()], MLA_SCALE)
        out = torch.from_numpy(ob[j:j + 1]).view(torch.bfloat16).float().numpy()
        lse = torch.from_numpy(lb[j:j + 1]).view(torch.float32).numpy()
        parity(out, lse, ro, rl, False, f"config5 batchmate {j} (len {L})")
