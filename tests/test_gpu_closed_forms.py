"""Closed forms of the attention definition, checked bit for bit on the GPU.

  * A row with one key (L = 1): the softmax weight is exactly 1, so the
    output is v_0; in bf16 output every kernel must return v_0's bits.
    (On the 128-head MLA path V enters the PV product as fp16, which holds
    every bf16 value of magnitude in [2^-14, 65504] exactly; the V values
    here are kept in that range.)
  * Rows whose keys all carry the same value vector v (powers of two, so
    every product p * v is exact): the output is v.  GQA's fp32 P path gives
    v's bits exactly; the MLA paths round P (fp16, or bf16 hi + lo) and must
    stay within one bf16 ulp.
  * q = 0: every score is 0, so the output is the mean of the values and
    the LSE is ln L (within the parity bar).

Each kernel family is reached through its own dispatch: Hq = 128 dense and
sparse MLA (the generated 128-head loop; the 32-heads-per-wave gather kernel
gives the same bits, checked in test_gpu_dense_kernels and
test_gpu_sparse_kernels), Hq = 64 MLA dense and sparse (16-head kernel) and
GQA.
"""

import math

import numpy as np
import pytest

from workloads import synth
from workloads.device import DeviceCase

from gpu_util import parity

pytestmark = pytest.mark.gpu

KERNELS = ["mla_h128_dense", "mla_h128_sparse", "mla_h64_dense", "mla_h64_sparse", "gqa_g4", "gqa_g1"]


def fp16_normal(bits):
    """bf16 bits with every magnitude below 2^-12 raised to 2^-12 (sign kept)."""
    x = synth.bf16_value(bits).astype(np.float32)
    small = np.abs(x) < 2.0 ** -12
    x[small] = np.where(x[small] < 0, -(2.0 ** -12), 2.0 ** -12)
    return synth.bf16_bits(x)


def make_case(kernel, lens, seed, topk=None):
    if kernel.startswith("gqa"):
        hkv = 2 if kernel == "gqa_g4" else 8
        return synth.gqa_case(lens, 8, hkv, 128, 1.0 / math.sqrt(128.0), 16, structure_seed=seed)
    hq = 128 if "h128" in kernel else 64
    sparse = kernel.endswith("sparse")
    case = synth.mla_case(lens, hq, 1.0 / math.sqrt(192.0), 64, structure_seed=seed,
                          topk_width=64 if sparse else 0, topk=topk if sparse else None)
    for r in case.rows:
        if sparse:
            r.gathered[:, :synth.MLA_DV] = fp16_normal(r.gathered[:, :synth.MLA_DV])
        else:
            r.latent[:, :synth.MLA_DV] = fp16_normal(r.latent[:, :synth.MLA_DV])
    return case


def values_of(case, b):
    """[L, heads-or-kv-heads, Dv] float32 value vectors of row b, key order."""
    r = case.rows[b]
    if isinstance(case, synth.GqaCase):
        return synth.bf16_value(r.v)
    lat = synth.bf16_value(r.gathered if case.sparse else r.latent)
    return lat[:, None, :synth.MLA_DV]


def head_map(case):
    """Value head of each query head."""
    if isinstance(case, synth.GqaCase):
        return np.arange(case.hq) // (case.hq // case.hkv)
    return np.zeros(case.hq, dtype=np.int64)


@pytest.mark.parametrize("kernel", KERNELS)
def test_single_key_rows_return_v0_bits(kernel):
    # dense: rows of length 1 among longer rows; sparse: every row attends one position
    lens = [1, 1, 300, 1, 2000, 1] if not kernel.endswith("sparse") else [1, 700, 5, 3000]
    case = make_case(kernel, lens, seed=71, topk=1)
    print(f"[case] L=1 closed form {kernel} lens={lens}", flush=True)
    dc = DeviceCase(case)
    dc.run()
    out, lse, bits, _ = dc.result()
    dc.close()
    hm = head_map(case)
    checked = 0
    for b in range(case.batch):
        n_keys = int(case.rows[b].topk_len) if getattr(case, "sparse", False) else int(case.lens[b])
        if n_keys != 1:
            continue
        v0 = values_of(case, b)[0][hm]                      # [Hq, Dv]
        want = synth.bf16_bits(v0).view(np.int16)
        assert np.array_equal(bits[b], want), f"{kernel}: row {b} (one key) is not v0 bit for bit"
        checked += 1
    assert checked >= 1


@pytest.mark.parametrize("kernel", KERNELS)
def test_equal_value_rows_return_v(kernel):
    sparse = kernel.endswith("sparse")
    lens = [7, 100, 1541, 3000] if not sparse else [7, 100, 1541, 3000]
    case = make_case(kernel, lens, seed=72, topk=None)
    rng = np.random.default_rng(73)
    wants = []
    for b, r in enumerate(case.rows):
        if isinstance(case, synth.GqaCase):
            v = (2.0 ** rng.integers(-3, 3, (case.hkv, case.d))) * rng.choice([-1.0, 1.0], (case.hkv, case.d))
            r.v[:] = synth.bf16_bits(v.astype(np.float32))[None]
        else:
            v = (2.0 ** rng.integers(-3, 3, synth.MLA_DV)) * rng.choice([-1.0, 1.0], synth.MLA_DV)
            vb = synth.bf16_bits(v.astype(np.float32))
            if sparse:
                r.gathered[:, :synth.MLA_DV] = vb[None]
            else:
                r.latent[:, :synth.MLA_DV] = vb[None]
        wants.append(values_of(case, b)[0][head_map(case)])
    print(f"[case] equal-V closed form {kernel} lens={lens}", flush=True)
    dc = DeviceCase(case)
    dc.run()
    out, lse, bits, _ = dc.result()
    dc.close()
    for b in range(case.batch):
        want = wants[b]
        if kernel.startswith("gqa"):
            assert np.array_equal(bits[b], synth.bf16_bits(want).view(np.int16)), f"{kernel}: row {b} is not v exactly"
        else:
            ulp = 2.0 ** (np.floor(np.log2(np.abs(want))) - 7)
            err = np.abs(out[b] - want)
            assert np.all(err <= ulp), f"{kernel}: row {b} off by {float((err / ulp).max()):.2f} bf16 ulp"


@pytest.mark.parametrize("kernel", KERNELS)
def test_zero_query_gives_the_mean_and_ln_length(kernel):
    sparse = kernel.endswith("sparse")
    lens = [3, 64, 1541, 5000] if not sparse else [40, 64, 1541, 5000]
    case = make_case(kernel, lens, seed=74, topk=None)
    for r in case.rows:
        r.q[:] = 0
    print(f"[case] q=0 closed form {kernel} lens={lens}", flush=True)
    dc = DeviceCase(case)
    dc.run()
    out, lse, _, _ = dc.result()
    dc.close()
    hm = head_map(case)
    ro = np.stack([values_of(case, b).astype(np.float64).mean(0)[hm] for b in range(case.batch)])
    n = [int(case.rows[b].topk_len) if sparse else int(case.lens[b]) for b in range(case.batch)]
    rl = np.stack([np.full(case.hq, math.log(k)) for k in n])
    parity(out, lse, ro, rl, False, f"q=0 {kernel}")


# ------------------------------------------------------------- fp16 V range

@pytest.mark.parametrize("hq", [128, 64])
def test_values_across_the_fp16_range(hq):
    """Latent V dims with magnitudes from 1e-7 to 6.5e4 (one scale per dim,
    log-uniform), so fp16 subnormals, the exact range and values next to the
    fp16 maximum all take part; the query's first 512 dims are zero, so the
    scores come from the rope dims alone and stay moderate.  Rows of 5, 300
    and 2000 tokens (the last with fp16 partials and the combine on the
    128-head path) against the oracle.

    Bar: the usual one, widened by the rounding of P (fp16, 2^-11 relative,
    or bf16 hi + lo) and of the partials, which a weighted sum passes on in
    proportion to sum_i w_i |v_i| -- not to |out|, which cancellation between
    large values of both signs can make far smaller:
        |gpu - ref| <= max(2e-3, ulp_bf16(ref), 2^-9 sum_i w_i |v_i|),
    sum_i w_i |v_i| being the oracle's output for |V| (the same weights,
    since V does not enter the scores here)."""
    import oracle
    from gpu_util import bf16_ulp, reference
    case = synth.mla_case([5, 300, 2000], hq, 1.0 / math.sqrt(192.0), 64, structure_seed=75)
    rng = np.random.default_rng(76)
    mag = np.exp(rng.uniform(math.log(1e-7), math.log(6.5e4), synth.MLA_DV)).astype(np.float32)
    for r in case.rows:
        v = synth.bf16_value(r.latent[:, :synth.MLA_DV]) * 2.0 * mag[None]    # N(0, 0.5) x 2 x scale
        v = np.clip(v, -65280.0, 65280.0)
        r.latent[:, :synth.MLA_DV] = synth.bf16_bits(v.astype(np.float32))
        r.q[:, :synth.MLA_DV] = 0
    print(f"[case] fp16 value range hq={hq}", flush=True)
    dc = DeviceCase(case, check_inputs=True)
    dc.run()
    out, lse, _, _ = dc.result()
    dc.close()
    ro, rl = reference(case)
    q = synth.bf16_value(case.q_bits())
    absrows = [np.concatenate([np.abs(x[:, :synth.MLA_DV]), x[:, synth.MLA_DV:]], axis=1)
               for x in case.logical_rows()]
    ra, _ = oracle.mla_decode(q, absrows, case.scale, dv=synth.MLA_DV)
    tol = np.maximum(np.maximum(2e-3, bf16_ulp(ro)), 2.0 ** -9 * ra)
    err = np.abs(out - ro)
    print(f"[parity] V range hq={hq}: max err/bar {float((err / tol).max()):.3f}, "
          f"max |out| {float(np.abs(ro).max()):.1f}", flush=True)
    assert np.all(err <= tol), f"{int((err > tol).sum())} elements outside the bar"
    assert np.max(np.abs(lse - rl)) <= 1e-3


@pytest.mark.parametrize("where", ["dense", "sparse"])
def test_check_inputs_reports_v_outside_fp16(where):
    """On the 128-head path an attended V value of 1e5 is reported as
    ISK_ERR_RANGE (row, position and dim named); the same value in a slot no
    row attends, or on the 16-head path, is accepted."""
    import invariant_split_kv_amd as isk
    big = synth.bf16_bits(np.array([1.0e5], np.float32))[0]
    for hq, attended, expect in ((128, True, -6), (128, False, 0), (64, True, 0)):
        if where == "dense":
            case = synth.mla_case([300, 200], hq, 0.1, 64, structure_seed=77)
            if attended:
                case.rows[1].latent[150, 33] = big
        else:
            case = synth.mla_case([900, 500], hq, 0.1, 64, structure_seed=78, topk_width=128)
            if attended:
                case.rows[1].gathered[7, 410] = big
        dc = DeviceCase(case, check_inputs=True)
        if not attended:
            # a slot past row 0's length on its last page (never attended)
            L0 = int(case.lens[0])
            slot = case.paging.token_slots(0, np.array([L0 - 1]))[0] + 1
            if slot % 64 != 0:
                dc.pool.view(-1, synth.MLA_DQK)[slot, 5] = torch_bf16(1.0e5)
        print(f"[case] range audit {where} hq={hq} attended={attended}", flush=True)
        if expect == 0:
            dc.run()
            dc.result()
        else:
            with pytest.raises(isk.IskError) as e:
                dc.run()
            assert e.value.status == expect and "row 1 position" in e.value.message, e.value.message
        dc.close()


def torch_bf16(x):
    import torch
    return torch.tensor(x, dtype=torch.bfloat16)
