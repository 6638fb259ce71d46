"""Parity of the HIP path against the fp64 oracle, through the C ABI.

Every configuration of the decode workloads runs at full size and is compared
element by element with the oracle; edge cases cover empty and one-token
rows, ragged tails at tile and split boundaries, garbage in unused cache
slots, sparse masking, other head counts and dims, and the input audit.
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

GARBAGE = int(synth.bf16_bits(np.array([3.0e4], np.float32))[0])   # finite, large


def run_case(case, **kw):
    print(f"[case] {type(case).__name__} B={case.batch} lens[:8]={list(case.lens[:8])} kw={kw}", flush=True)
    dc = DeviceCase(case, **kw)
    dc.run()
    out, lse, bits, lbits = dc.result()
    dc.close()
    return out, lse, bits, lbits


@pytest.mark.parametrize("out_f32", [False, True])
def test_config1_gqa_tiny(out_f32):
    case = synth.config1_gqa_tiny()
    out, lse, _, _ = run_case(case, out_f32=out_f32)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, out_f32, f"config1 out_f32={out_f32}")


def test_config2_gqa_llama8b_shape():
    case = synth.config2_gqa()
    out, lse, _, _ = run_case(case)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, "config2")


@pytest.mark.parametrize("out_f32", [False, True])
def test_config3_mla(out_f32):
    case = synth.config3_mla()
    out, lse, _, _ = run_case(case, out_f32=out_f32)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, out_f32, f"config3 out_f32={out_f32}")


def test_config4_sparse_mla():
    case = synth.config4_sparse()
    out, lse, _, _ = run_case(case)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, "config4")


@pytest.mark.parametrize("mode", [isk.SPLIT_PER_ROW, isk.SPLIT_BATCH_BALANCED])
def test_balanced_mode_parity(mode):
    case = synth.config3_mla(batch=16)
    out, lse, _, _ = run_case(case, split_mode=mode)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, f"config3 B=16 mode={mode}")


# ---------------------------------------------------------------- edge cases

EDGE_LENS = [0, 1, 2, 63, 64, 65, 511, 512, 513, 1023, 1024, 1025, 2100]


@pytest.mark.parametrize("g,d", [(4, 128), (1, 64), (2, 128), (8, 64), (8, 128), (16, 128)])
def test_gqa_edges_and_group_sizes(g, d):
    hkv = 2
    case = synth.gqa_case(EDGE_LENS, g * hkv, hkv, d, 1.0 / math.sqrt(d), 16, structure_seed=30 + g)
    out, lse, _, _ = run_case(case, fill=GARBAGE)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, f"gqa edges g={g} d={d}")


@pytest.mark.parametrize("hq", [128, 256, 64, 48, 32, 16])
def test_mla_edges_and_head_counts(hq):
    case = synth.mla_case(EDGE_LENS, hq, 1.0 / math.sqrt(192.0), 64, structure_seed=40 + hq)
    out, lse, _, _ = run_case(case, fill=GARBAGE)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, f"mla edges hq={hq}")


def test_mla_page_size_128_and_custom_split():
    case = synth.mla_case([3000, 129, 5000, 64], 128, 0.07, 128, structure_seed=50, split_tokens=256)
    out, lse, _, _ = run_case(case)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, "mla P=128 S=256")


@pytest.mark.parametrize("hq,out_f32", [(128, False), (128, True), (64, False)])
def test_combine_over_64_splits(hq, out_f32):
    """Rows with more than 64 splits (79 and 313 at S = 64) take the
    combine's chunked path (LSEs loaded 64 at a time, then chained); fp16
    partials (128 heads, bf16 output) and fp32 partials (fp32 output, or the
    16-head kernel) both go through it."""
    case = synth.mla_case([5000, 20000, 70, 1], hq, 0.07, 64, structure_seed=53, split_tokens=64)
    out, lse, _, _ = run_case(case, out_f32=out_f32)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, out_f32, f"mla >64 splits hq={hq} f32={out_f32}")


def _grow_rope_scores(case, growth):
    """Scale the 64 rope dims of each cached token by growth(t / L): the
    scores climb (or jump) across the row while the values (the first 512
    dims) keep their N(0, 0.5^2) range, so the tolerance stays tight."""
    for b, r in enumerate(case.rows):
        L = int(case.lens[b])
        if L == 0:
            continue
        g = np.asarray(growth(np.arange(L) / max(L - 1, 1)), np.float32)[:, None]
        rope = synth.bf16_value(r.latent[:, 512:]) * g
        r.latent[:, 512:] = synth.bf16_bits(rope)
    return case


@pytest.mark.parametrize("hq", [128, 64])
@pytest.mark.parametrize("shape", ["ramp", "jump"])
def test_mla_running_max_moves_rescale_accumulator(hq, shape):
    """Rows whose scores grow far past the lazy-rescale threshold (2^8 in
    the exponent) several times per split, so the accumulator rescale runs;
    the normal workloads' flat scores never trigger it."""
    growth = (lambda x: 1.0 + 200.0 * x) if shape == "ramp" else (lambda x: np.where(x < 0.6, 1.0, 150.0))
    case = _grow_rope_scores(synth.mla_case([3000, 5000, 700, 64, 1537], hq, 1.0 / math.sqrt(192.0), 64,
                                            structure_seed=70 + hq), growth)
    for out_f32 in (False, True):
        out, lse, _, _ = run_case(case, out_f32=out_f32)
        ro, rl = reference(case)
        parity(out, lse, ro, rl, out_f32, f"mla rescale {shape} hq={hq} f32={out_f32}")


@pytest.mark.parametrize("hq", [128, 64])
def test_mla_split_longer_than_the_page_window(hq):
    """Splits of 8192 tokens over 64-token pages span 128 pages: tiles past
    the first 64 pages of a split read the block table directly."""
    case = synth.mla_case([9000, 20000, 8192], hq, 1.0 / math.sqrt(192.0), 64, structure_seed=80 + hq,
                          split_tokens=8192)
    out, lse, _, _ = run_case(case, fill=GARBAGE)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, f"mla S=8192 hq={hq}")


def test_sparse_edges():
    W = 700
    lens = [3000, 5, 800, 2000, 1, 0, 4096]
    case = synth.mla_case(lens, 128, 1.0 / math.sqrt(192.0), 64, structure_seed=60, topk_width=W)
    rows = case.rows
    rng = np.random.default_rng(61)
    rows[0].topk_idx[[3, 10, 200]] = -1                  # -1 inside topk_len: skipped
    rows[2].topk_idx[[0, 1]] = [900, 100000]             # >= len: skipped
    rows[3].topk_idx[5] = rows[3].topk_idx[6]            # duplicate position counts twice
    rows[3].gathered[5] = rows[3].gathered[6]
    rows[6].topk_len = 513                               # shorter than the row's entries
    rows[6].topk_idx[513:] = rng.integers(0, 4096, W - 513)
    out, lse, _, _ = run_case(case, fill=GARBAGE)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, "sparse edges")
    assert np.all(out[5] == 0) and np.all(np.isneginf(lse[5]))


@pytest.mark.parametrize("hq", [128, 64])
def test_sparse_device_length_beyond_the_table_is_clamped(hq):
    """A device length above max_pages_per_row * page_size (the plan saw the
    true length; inputs are not audited) does not let a top-k position past
    the row's block table through: such positions are masked like positions
    past the length.  (The positions used stay below twice the cap, so even
    an unclamped read would stay inside the block-table allocation.)"""
    case = synth.mla_case([600, 300], hq, 0.1, 64, structure_seed=67, topk_width=256)
    cap = case.paging.max_pages_per_row * 64
    assert cap == 640
    case.rows[0].topk_idx[[2, 50, 100]] = [700, cap, 2 * cap - 1]   # past the table (and the length)
    dc = DeviceCase(case, fill=GARBAGE)
    dc.lens[0] = 2 * cap - 40                                        # device length past the table
    dc.run()
    out, lse, _, _ = dc.result()
    dc.close()
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, f"sparse device length past the table hq={hq}")


def test_all_masked_sparse_row_gives_zero_and_neg_inf():
    case = synth.mla_case([100, 50], 64, 0.1, 64, structure_seed=62, topk_width=128)
    case.rows[0].topk_idx[:] = -1
    out, lse, _, _ = run_case(case)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, "sparse all-masked")


def test_check_inputs_reports_bad_tables():
    case = synth.mla_case([300, 200], 64, 0.1, 64, structure_seed=63, topk_width=64)
    case.rows[1].topk_idx[3] = 250                       # >= len inside topk_len
    dc = DeviceCase(case, check_inputs=True)
    with pytest.raises(isk.IskError) as e:
        dc.run()
    assert e.value.status == -4 and "topk_idx[1][3]" in e.value.message
    dc.close()
    # A block-table entry outside the pool, set on the device copy only (the
    # pool itself is staged from the valid table).
    dense = synth.mla_case([300, 200], 64, 0.1, 64, structure_seed=64)
    dc = DeviceCase(dense, check_inputs=True)
    dc.block_table[0, 2] = dense.paging.num_pages + 5
    with pytest.raises(isk.IskError) as e:
        dc.run()
    assert e.value.status == -4 and "block_table[0][2]" in e.value.message
    dc.close()
    good = DeviceCase(synth.mla_case([300, 200], 64, 0.1, 64, structure_seed=65), check_inputs=True)
    good.run()
    good.close()


def test_out_of_pool_page_is_masked_not_read():
    """Without the audit, a block-table entry outside the pool masks its
    tokens instead of being dereferenced."""
    case = synth.mla_case([300, 200], 64, 0.1, 64, structure_seed=66)
    dc = DeviceCase(case)
    dc.block_table[0, 1] = case.paging.num_pages + 1000   # tokens 64..127 of row 0
    dc.run()
    out, lse, _, _ = dc.result()
    dc.close()
    keep = np.r_[0:64, 128:300]
    row0 = synth.bf16_value(case.rows[0].latent)[keep]
    q = synth.bf16_value(case.q_bits())
    import oracle
    ro0, rl0 = oracle.mla_decode(q[:1], [row0], case.scale)
    parity(out[:1], lse[:1], ro0, rl0, False, "masked page")


@pytest.mark.parametrize("kind", ["gqa", "mla", "sparse"])
def test_oneshot_entry_matches_planned_call(kind):
    """isk_attn_decode_oneshot (plan + stream-ordered workspace + decode in one
    call) gives the bits of the plan-based call and passes parity itself."""
    if kind == "gqa":
        case = synth.config1_gqa_tiny()
    elif kind == "mla":
        case = synth.mla_case([1, 100, 1537, 3100], 128, 1 / math.sqrt(192.0), 64, structure_seed=71)
    else:
        case = synth.mla_case([300, 2500, 64], 128, 1 / math.sqrt(192.0), 64, structure_seed=72,
                              topk_width=1024)
    print(f"[oneshot] {kind} B={case.batch} lens={list(case.lens)}", flush=True)
    dc = DeviceCase(case)
    dc.run()
    _, _, bits, lbits = dc.result()
    out2 = torch.empty_like(dc.out)
    lse2 = torch.empty_like(dc.lse)
    isk.attn_decode_oneshot(dc.desc, dc.lens_host, dc.topk_len_host, dc.q, dc.pool, dc.block_table, dc.lens,
                            dc.topk_idx, dc.topk_len, out2, lse2)
    torch.cuda.synchronize()
    assert np.array_equal(out2.view(torch.int16).cpu().numpy(), bits)
    assert np.array_equal(lse2.view(torch.int32).cpu().numpy(), lbits)
    ro, rl = reference(case)
    parity(out2.float().cpu().numpy().astype(np.float64), lse2.cpu().numpy().astype(np.float64), ro, rl, False,
           f"oneshot {kind}")
    dc.close()


# ----------------------------------------------------------------------------
# Extra KV source (a second gathered set per row, from its own cache)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("out_f32", [False, True])
def test_sparse_extra_source(out_f32):
    case = synth.config4_sparse_extra()
    out, lse, _, _ = run_case(case, out_f32=out_f32)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, out_f32, f"sparse + extra out_f32={out_f32}")


def test_sparse_extra_source_edges():
    """Either set empty, both empty, masked extra slots, an extra set of three
    splits, a smaller extra page size, garbage in unused slots."""
    lens = [3000, 900, 50, 4000, 2500, 6000]
    xlens = [400, 2000, 0, 9, 1500, 3000]
    XW = 1100
    case = synth.mla_extra_case(lens, xlens, 128, 1.0 / math.sqrt(192.0), 64, structure_seed=70,
                                topk_width=700, extra_width=XW, extra_page_size=16)
    rows, xrows = case.rows, case.extra.rows
    xrows[0].topk_len = 0                                # extra set empty
    rows[1].topk_len = 0                                 # main set empty
    rows[2].topk_len = 0                                 # both empty (extra len 0)
    xrows[4].topk_idx[[0, 7, 300]] = -1                  # -1 inside the extra topk_len
    xrows[4].topk_idx[[1, 2]] = [1500, 99999]            # >= extra len: skipped
    xrows[5].topk_len = 1100                             # three extra splits of 512
    out, lse, _, _ = run_case(case, fill=GARBAGE)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, "sparse + extra edges")
    assert np.all(out[2] == 0) and np.all(np.isneginf(lse[2]))


def test_sparse_extra_source_audit():
    case = synth.mla_extra_case([300, 200], [100, 50], 64, 0.1, 64, structure_seed=71, topk_width=64,
                                extra_width=32)
    case.extra.rows[1].topk_idx[4] = 60                  # >= extra len 50 inside the extra topk_len
    dc = DeviceCase(case, check_inputs=True)
    with pytest.raises(isk.IskError) as e:
        dc.run()
    assert e.value.status == -4 and "extra topk_idx[1][4]" in e.value.message
    dc.close()
    good = DeviceCase(synth.mla_extra_case([300, 200], [100, 50], 64, 0.1, 64, structure_seed=72, topk_width=64,
                                           extra_width=32), check_inputs=True)
    good.run()
    good.close()


def test_sparse_extra_source_16_head_kernel():
    case = synth.mla_extra_case([3000, 700, 5000], [900, 30, 2000], 64, 1.0 / math.sqrt(192.0), 64,
                                structure_seed=73, topk_width=600, extra_width=700)
    out, lse, _, _ = run_case(case)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, "sparse + extra, 64 heads")


# ----------------------------------------------------------------------------
# Plans passed in the kernel arguments (dense per-row plans of at most 640
# splits and 128 rows) and plans uploaded through the workspace
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("rows,split", [(128, 1536), (129, 1536), (40, 64)])
def test_plans_by_value_and_uploaded_at_the_size_limits(rows, split):
    """128 rows fit the by-value plan, 129 do not; 40 rows of up to 2600
    tokens with 64-token splits need more than 640 splits (uploaded)."""
    rng = np.random.default_rng(80 + rows)
    lens = rng.integers(0, 2600 if split == 64 else 3000, rows)
    lens[:3] = [0, 1, 1536]
    case = synth.mla_case(lens, 128, 1.0 / math.sqrt(192.0), 64, structure_seed=81 + rows, split_tokens=split)
    n_splits = int(sum(-(-int(L) // split) for L in lens))
    print(f"[case] rows={rows} splits={n_splits}", flush=True)
    out, lse, _, _ = run_case(case)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, f"plan size rows={rows} splits={n_splits}")
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


def test_gqa_plan_by_value_matches_uploaded_plan_bits():
    """The same GQA rows decoded as a by-value plan (32 rows) and inside an
    uploaded plan (the rows repeated to 160) give identical bits."""
    small = synth.config2_gqa()
    _, _, bits_small, lbits_small = run_case(small)
    big_lens = np.concatenate([small.lens] * 5)
    paging = synth.make_paging(big_lens, 16, np.random.default_rng(82))
    big = synth.GqaCase(small.rows * 5, big_lens, 32, 8, 128, small.scale, paging)
    _, _, bits_big, lbits_big = run_case(big)
    for k in range(5):
        sl = slice(32 * k, 32 * (k + 1))
        assert np.array_equal(bits_big[sl], bits_small) and np.array_equal(lbits_big[sl], lbits_small)


@pytest.mark.parametrize("hq", [128, 64])
def test_sparse_segments_longer_than_the_row_window(hq):
    """Sparse splits of 3072 slots: the 128-head kernel resolves pool rows in
    windows of 1024 slots, so these segments move the window twice.  Masked
    slots sit at window boundaries; one segment ends inside a window."""
    W = 3000
    lens = [70000, 5000, 2999]
    case = synth.mla_case(lens, hq, 1.0 / math.sqrt(192.0), 64, structure_seed=90, topk_width=W,
                          split_tokens=3072)
    rows = case.rows
    rows[0].topk_idx[[1023, 1024, 2047, 2048, 2999]] = -1          # at the window edges
    rows[1].topk_idx[[0, 1500]] = [70000, 5000]                    # >= len: skipped
    rows[2].topk_len = 2100                                        # ends inside the third window
    out, lse, _, _ = run_case(case, fill=GARBAGE)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, f"sparse 3072-slot splits hq={hq}")


@pytest.mark.parametrize("which", ["gqa", "mla"])
def test_timing_hook_launch_gives_the_same_bits(which):
    """With timing events set, the split kernel goes through
    hipExtLaunchKernel; its output bits equal the plain launch's and the
    events bracket a positive kernel time."""
    import ctypes
    rt = ctypes.CDLL("libamdhip64.so")   # the runtime torch (and libisk) already use
    rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
    case = synth.config1_gqa_tiny() if which == "gqa" else synth.config3_mla(batch=8)
    dc = DeviceCase(case)
    dc.run()
    _, _, bits0, lbits0 = dc.result()
    evs = []
    for _ in range(3):
        e = ctypes.c_void_p()
        assert rt.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    isk.plan_set_timing_events(dc.plan.handle, *evs)
    dc.run()
    _, _, bits1, lbits1 = dc.result()
    isk.plan_set_timing_events(dc.plan.handle, None, None, None)
    ms = ctypes.c_float()
    assert rt.hipEventSynchronize(evs[2]) == 0
    assert rt.hipEventElapsedTime(ctypes.byref(ms), evs[0], evs[1]) == 0 and ms.value > 0.0
    assert rt.hipEventElapsedTime(ctypes.byref(ms), evs[1], evs[2]) == 0 and ms.value >= 0.0
    for e in evs:
        rt.hipEventDestroy(e)
    dc.close()
    assert np.array_equal(bits0, bits1) and np.array_equal(lbits0, lbits1)


@pytest.mark.parametrize("nbytes,blocks", [(1 << 20, 64), ((1 << 24) + 48, 1000), (4096 * 16, 4096)])
def test_hbm_read_probe_reads_every_word_once(nbytes, blocks):
    """The streaming-read probe behind the measured HBM read peak folds every
    32-bit word of its buffer into the per-workgroup XOR words exactly once
    (a word read twice, or not at all, changes the fold)."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), generator=g, device="cuda", dtype=torch.int32)
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    isk.hbm_read_probe(buf, nbytes, sink, blocks)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("n_rows,row_bytes,blocks", [(1, 1152, 1), (777, 1152, 64), (5000, 1152, 1024), (300, 16, 7)])
def test_hbm_gather_probe_reads_every_listed_row_once(n_rows, row_bytes, blocks):
    """The gather probe behind the sparse path's measured ceiling folds every
    32-bit word of every listed row (repeats included) into the per-workgroup
    XOR words exactly once."""
    import torch
    rng = np.random.default_rng(n_rows)
    pool_rows = 4096
    pool = rng.integers(0, 2 ** 32, (pool_rows, row_bytes // 4), dtype=np.uint64).astype(np.uint32)
    rows = rng.integers(0, pool_rows, n_rows).astype(np.int32)
    buf = torch.from_numpy(pool.view(np.int32)).cuda()
    rows_d = torch.from_numpy(rows).cuda()
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    isk.hbm_gather_probe(buf, pool.nbytes, rows_d, n_rows, row_bytes, sink, blocks)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(pool[rows].reshape(-1)) if n_rows else 0
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


def test_sparse_plan_by_value_matches_uploaded_plan_bits():
    """The same sparse rows decoded as a by-value plan (40 rows: split ranges
    rebuilt in the kernels from the device top-k counts) and inside an
    uploaded plan (the rows repeated to 160) give identical bits; both run
    the generated 128-head loop."""
    small = synth.mla_case(np.random.default_rng(130).integers(1, 5000, 40), 128, 1.0 / math.sqrt(192.0), 64,
                           structure_seed=131, topk_width=1024)
    small.rows[3].topk_len = 700                       # a row shorter than its entries
    small.rows[5].topk_idx[:40] = -1
    _, _, bits_small, lbits_small = run_case(small)
    big_lens = np.concatenate([small.lens] * 4)
    paging = synth.make_paging(big_lens, 64, np.random.default_rng(132))
    big = synth.MlaCase(small.rows * 4, big_lens, 128, small.scale, paging, small.topk_width)
    _, _, bits_big, lbits_big = run_case(big)
    for k in range(4):
        sl = slice(40 * k, 40 * (k + 1))
        assert np.array_equal(bits_big[sl], bits_small) and np.array_equal(lbits_big[sl], lbits_small)
