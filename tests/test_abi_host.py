"""Host-side checks of the C ABI: the library loads, exports what the header
declares, validates arguments, and plans splits as specified.  No kernel runs.

Per-row split rule (FlashMLA issue page "Sparse MLA decode is not
batch-invariant ...", section "Question"): a row's splits derive from its
own length and fixed constants only.  The batch-balanced comparison mode
(same page, section "Where it comes from") derives them from batch totals.
"""
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import invariant_split_kv_amd as isk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def gqa_desc(**kw):
    d = dict(kind=isk.KIND_GQA, num_q_heads=32, num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=16,
             num_pages=100000, max_pages_per_row=8192, topk_width=0, split_mode=isk.SPLIT_PER_ROW,
             split_tokens=0, out_dtype=isk.OUT_BF16, check_inputs=0, scale=0.088)
    d.update(kw)
    return isk.IskDesc(**d)


def mla_desc(**kw):
    d = dict(kind=isk.KIND_MLA, num_q_heads=128, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=64,
             num_pages=100000, max_pages_per_row=2048, topk_width=0, split_mode=isk.SPLIT_PER_ROW,
             split_tokens=0, out_dtype=isk.OUT_BF16, check_inputs=0, scale=0.072)
    d.update(kw)
    return isk.IskDesc(**d)


def segments(desc, lens, topk=None):
    with isk.Plan(desc, lens, topk) as p:
        return p.segments(), p.info()


def test_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "isk.h")).read()
    declared = set(re.findall(r"ISK_API\s+[\w\s\*]+?\b(isk_\w+)\s*\(", header))
    assert len(declared) == 19
    for name in declared:
        assert hasattr(isk.lib, name), name
    assert "gfx950" in isk.numerics_id()


def test_invalid_arguments_are_rejected_with_status_and_message():
    cases = [
        (gqa_desc(num_q_heads=30), [5], -1, "multiple"),
        (gqa_desc(num_q_heads=24, num_kv_heads=8), [5], -2, "group size"),
        (gqa_desc(head_dim_qk=96, head_dim_v=96), [5], -2, "head_dim"),
        (gqa_desc(split_tokens=100), [5], -1, "split_tokens"),
        (gqa_desc(split_mode=7), [5], -1, "split_mode"),
        (gqa_desc(), [16 * 8192 + 1], -1, "outside"),
        (gqa_desc(), [-1], -1, "outside"),
        (mla_desc(num_kv_heads=2), [5], -1, "latent"),
        (mla_desc(num_q_heads=96), [5], -2, "multiple of 16"),
        (mla_desc(page_size=16), [5], -2, "page_size"),
        (mla_desc(num_pages=2 ** 25), [5], -2, "2^31"),            # 2^25 pages x 64 rows = 2^31 rows
        (mla_desc(max_pages_per_row=2 ** 25), [5], -2, "int32"),   # a row table of 2^31 token positions
        (gqa_desc(topk_width=16), [5], -2, "MLA only"),
        (gqa_desc(scale=float("nan")), [5], -1, "finite"),
        (gqa_desc(scale=0.0), [5], -1, "positive"),
        (gqa_desc(scale=-0.1), [5], -1, "positive"),
    ]
    for desc, lens, status, text in cases:
        with pytest.raises(isk.IskError) as e:
            isk.plan_create(desc, lens)
        assert e.value.status == status and text in e.value.message, (e.value.status, e.value.message)
    with pytest.raises(isk.IskError) as e:
        isk.plan_create(mla_desc(topk_width=64), [100])          # sparse needs topk_len_host
    assert e.value.status == -1
    with pytest.raises(isk.IskError) as e:
        isk.plan_create(mla_desc(), [100], [5])                  # dense must not get one
    assert e.value.status == -1


def test_decode_argument_errors_without_launch():
    desc = gqa_desc()
    with isk.Plan(desc, [100, 7]) as p:
        ws = p.workspace_bytes
        with pytest.raises(isk.IskError) as e:   # workspace too small: rejected before any HIP call
            isk.attn_decode(p.handle, 256, 256, 256, 256, None, None, 256, 256, 256, ws - 1, stream=0)
        assert e.value.status == -3
        with pytest.raises(isk.IskError) as e:   # NULL q
            isk.attn_decode(p.handle, None, 256, 256, 256, None, None, 256, 256, 256, ws, stream=0)
        assert e.value.status == -1
        with pytest.raises(isk.IskError) as e:   # dense plan given top-k arrays
            isk.attn_decode(p.handle, 256, 256, 256, 256, 256, 256, 256, 256, 256, ws, stream=0)
        assert e.value.status == -1
        with pytest.raises(isk.IskError) as e:   # misaligned workspace
            isk.attn_decode(p.handle, 256, 256, 256, 256, None, None, 256, 256, 260, ws, stream=0)
        assert e.value.status == -3
    # The one-shot entry checks its arguments before allocating anything.
    with pytest.raises(isk.IskError) as e:
        isk.attn_decode_oneshot(desc, [100, 7], None, None, 256, 256, 256, 256, None, 256, 256, stream=0)
    assert e.value.status == -1 and "non-NULL" in e.value.message
    with pytest.raises(isk.IskError) as e:
        isk.attn_decode_oneshot(gqa_desc(num_q_heads=30), [5], None, 256, 256, 256, 256, None, None, 256, 256,
                                stream=0)
    assert e.value.status == -1 and "multiple" in e.value.message


def _check_tiling(segs, info, units, split):
    by_row = {}
    for r, b, e, part, g in segs:
        by_row.setdefault(r, []).append((b, e, part))
    slots = []
    for r, U in enumerate(units):
        pieces = sorted(by_row.get(r, []))
        if U == 0:
            assert not pieces
            continue
        assert pieces[0][0] == 0 and pieces[-1][1] == U
        for (b0, e0, _), (b1, _, _) in zip(pieces[:-1], pieces[1:]):
            assert e0 == b1
        for b, e, part in pieces:
            assert e > b and b % 64 == 0
        if len(pieces) == 1:
            assert pieces[0][2] == -1
        else:
            parts = [p for _, _, p in pieces]
            assert parts == list(range(parts[0], parts[0] + len(parts)))
            slots += parts
    assert len(slots) == len(set(slots)) == info["num_partials"]
    if split is not None:
        for r, U in enumerate(units):
            assert len(by_row.get(r, [])) == -(-U // split)


def test_per_row_plan_matches_formula_config_shapes():
    lens = [17, 100, 256, 1000, 0, 1, 64, 65]
    segs, info = segments(gqa_desc(split_tokens=64, num_q_heads=8, num_kv_heads=2, head_dim_qk=64,
                                   head_dim_v=64, page_size=64), lens)
    _check_tiling(segs, info, lens, 64)
    assert info["num_segments"] == sum(-(-L // 64) for L in lens)
    # longest splits are dispatched first, in blocks of 32 tasks
    lengths = segs[:, 2] - segs[:, 1]
    blocks = [lengths[i:i + 32] for i in range(0, len(lengths), 32)]
    assert all(a.min() >= b.max() for a, b in zip(blocks, blocks[1:]))


def test_per_row_launch_order_puts_a_rows_splits_on_one_xcd():
    """Task t runs on XCD t % 8; in each full block of 32 tasks XCD x takes
    sorted tasks 4x .. 4x+3, so the four 512-slot splits of a sparse
    2048-slot row share one XCD."""
    tl = [2048] * 16
    segs, info = segments(mla_desc(topk_width=2048), [70000] * 16, tl)
    assert info["num_segments"] == 64
    for r in range(16):
        tasks = [t for t in range(64) if segs[t, 0] == r]
        assert len(tasks) == 4 and len({t % 8 for t in tasks}) == 1, (r, tasks)


def test_sparse_plan_uses_topk_len():
    topk = [2048, 0, 5, 3000, -4]
    lens = [4000, 10, 10, 70000, 9]
    segs, info = segments(mla_desc(topk_width=2048, max_pages_per_row=2048), lens, topk)
    units = [2048, 0, 5, 2048, 0]
    _check_tiling(segs, info, units, 512)


@settings(max_examples=80, deadline=None)
@given(lens=st.lists(st.integers(0, 20000), min_size=1, max_size=24), probe=st.integers(0, 20000),
       pos=st.integers(0, 24), mla=st.booleans())
def test_per_row_splits_do_not_depend_on_batchmates(lens, probe, pos, mla):
    desc = mla_desc(max_pages_per_row=512) if mla else gqa_desc(max_pages_per_row=2048)
    solo, _ = segments(desc, [probe])
    pos = min(pos, len(lens))
    batch = lens[:pos] + [probe] + lens[pos:]
    segs, info = segments(desc, batch)
    _check_tiling(segs, info, batch, info["split_tokens"])
    mine = sorted((b, e) for r, b, e, _, _ in segs if r == pos)
    assert mine == sorted((b, e) for _, b, e, _, _ in solo)


@settings(max_examples=40, deadline=None)
@given(lens=st.lists(st.integers(0, 40000), min_size=1, max_size=40))
def test_balanced_plan_tiles_rows(lens):
    segs, info = segments(mla_desc(split_mode=isk.SPLIT_BATCH_BALANCED, max_pages_per_row=1024), lens)
    _check_tiling(segs, info, lens, None)
    groups = segs[:, 4]
    assert np.all(np.diff(groups) >= 0)


def test_balanced_plan_depends_on_batchmates():
    """Negative control: the batch-wide quota moves a row's split points."""
    desc = mla_desc(split_mode=isk.SPLIT_BATCH_BALANCED)
    probe = 16384
    seen = set()
    for mates in ([], [1000], [131072, 131072], [5000] * 31, [70000] * 127):
        segs, _ = segments(desc, [probe] + mates)
        seen.add(tuple(sorted((int(b), int(e)) for r, b, e, _, _ in segs if r == 0)))
    assert len(seen) >= 3


def test_workspace_size_covers_partials():
    lens = [5000, 3000, 100]
    with isk.Plan(mla_desc(), lens) as p:
        info = p.info()
        S = info["split_tokens"]
        expect = sum(-(-L // S) for L in lens if -(-L // S) > 1)   # rows with one split need no partial
        assert info["num_partials"] == expect > 0
        # 128-head MLA with bf16 output: fp16 partials (2 bytes) and fp32 LSEs
        assert info["workspace_bytes"] >= expect * 128 * (512 * 2 + 4)
        assert p.workspace_bytes == info["workspace_bytes"]
    with isk.Plan(mla_desc(out_dtype=isk.OUT_F32), lens) as p:   # fp32 output: fp32 partials
        assert p.info()["workspace_bytes"] >= expect * 128 * (512 + 1) * 4
    with isk.Plan(mla_desc(num_q_heads=64), lens) as p:           # 16-head kernel: fp32 partials
        assert p.info()["workspace_bytes"] >= expect * 64 * (512 + 1) * 4
    with isk.Plan(mla_desc(), lens) as p:
        p.update([100, 100])
        assert p.info()["num_partials"] == 0 and p.info()["batch"] == 2


# ----------------------------------------------------------------------------
# Extra KV source (sparse MLA): planner and argument checks
# ----------------------------------------------------------------------------

def xdesc(**kw):
    d = dict(page_size=64, num_pages=4096, max_pages_per_row=256, topk_width=1024)
    d.update(kw)
    return isk.IskExtraDesc(**d)


def extra_segments(lens, tl, xtl, width=2048, xwidth=1024, split=0):
    with isk.Plan(mla_desc(topk_width=width, split_tokens=split), lens, tl, extra=xdesc(topk_width=xwidth),
                  extra_topk_len_host=xtl) as p:
        return p.segments(), p.info()


def test_extra_source_splits_follow_the_main_splits_per_row():
    W, S = 2048, 512
    segs, info = extra_segments([5000, 100, 9000], [2048, 0, 700], [900, 1024, 0])
    by_row = {}
    for r in segs:
        by_row.setdefault(int(r[0]), []).append(r)
    for b, (n_main, xtl) in enumerate([(4, 900), (0, 1024), (2, 0)]):
        rs = sorted(by_row.get(b, []), key=lambda r: r[3] if r[3] >= 0 else 0)
        main = [r for r in rs if r[1] < W]
        extra = [r for r in rs if r[1] >= W]
        assert len(main) == n_main
        assert [(int(r[1]) - W, int(r[2]) - W) for r in sorted(extra, key=lambda r: r[1])] == \
            [(i * S, min((i + 1) * S, xtl)) for i in range(-(-xtl // S))]
        # partial slots: the row's main splits first, then its extra splits
        if len(rs) > 1:
            slots = [int(r[3]) for r in sorted(main, key=lambda r: r[1])] + \
                    [int(r[3]) for r in sorted(extra, key=lambda r: r[1])]
            assert slots == list(range(slots[0], slots[0] + len(slots)))
    assert info["num_segments"] == 4 + 0 + 2 + 2 + 2 + 0


@settings(max_examples=40, deadline=None)
@given(xtl=st.lists(st.integers(-3, 1300), min_size=1, max_size=8), seed=st.integers(0, 2 ** 31 - 1))
def test_extra_splits_of_a_row_do_not_depend_on_batchmates(xtl, seed):
    rng = np.random.default_rng(seed)
    B = len(xtl)
    lens = rng.integers(1, 70000, B)
    tl = rng.integers(0, 2049, B)
    segs, _ = extra_segments(lens, tl, xtl)
    for b in range(B):
        solo, _ = extra_segments([lens[b]], [tl[b]], [xtl[b]])
        mine = sorted((int(r[1]), int(r[2])) for r in segs if r[0] == b)
        assert mine == sorted((int(r[1]), int(r[2])) for r in solo)


def test_extra_source_arguments_are_checked():
    bad = [
        (dict(), dict(page_size=0), -1, "positive"),
        (dict(), dict(topk_width=0), -1, "positive"),
        (dict(), dict(num_pages=2 ** 26, page_size=64), -2, "2^31"),
        (dict(topk_width=0), dict(), -2, "sparse MLA"),
        (dict(split_mode=isk.SPLIT_BATCH_BALANCED), dict(), -2, "per-row"),
    ]
    for dkw, xkw, status, text in bad:
        with pytest.raises(isk.IskError) as e:
            isk.plan_create_extra(mla_desc(**{"topk_width": 2048, **dkw}), xdesc(**xkw), [100], [10], [5])
        assert e.value.status == status and text in e.value.message, (e.value.status, e.value.message)
    with pytest.raises(isk.IskError) as e:
        isk.plan_create_extra(mla_desc(topk_width=2048), xdesc(), [100], [10], None)
    assert e.value.status == -1 and "extra_topk_len_host" in e.value.message
    # an extra plan is not re-planned in place
    with isk.Plan(mla_desc(topk_width=2048), [100], [10], extra=xdesc(), extra_topk_len_host=[5]) as p:
        with pytest.raises(isk.IskError) as e:
            p.update([200], [20])
        assert e.value.status == -1 and "isk_plan_create_extra" in e.value.message


def test_decode_entry_points_match_the_plan_kind():
    # Mismatches are rejected before any device work (fake, aligned addresses).
    A = 1 << 20
    with isk.Plan(mla_desc(topk_width=2048), [100], [10], extra=xdesc(), extra_topk_len_host=[5]) as p:
        with pytest.raises(isk.IskError) as e:
            isk.attn_decode(p.handle, A, A, A, A, A, A, A, A, A, p.workspace_bytes, 0)
        assert "isk_attn_decode_extra" in e.value.message
        with pytest.raises(isk.IskError) as e:
            isk.attn_decode_extra(p.handle, A, A, A, A, A, A, A, None, A, A, A, A, A, A, p.workspace_bytes, 0)
        assert e.value.status == -1 and "non-NULL" in e.value.message
    with isk.Plan(mla_desc(topk_width=2048), [100], [10]) as p:
        with pytest.raises(isk.IskError) as e:
            isk.attn_decode_extra(p.handle, A, A, A, A, A, A, A, A, A, A, A, A, A, A, p.workspace_bytes, 0)
        assert "no extra KV source" in e.value.message


def test_rmsnorm_arguments_are_checked_before_any_device_work():
    A = 1 << 20
    bad = [(-1, 64, 1e-6, -1, "rows"), (4, 12, 1e-6, -2, "multiple of 8"), (4, 16392, 1e-6, -2, "multiple of 8"),
           (4, 0, 1e-6, -2, "multiple of 8"), (4, 64, float("nan"), -1, "eps"), (4, 64, -1.0, -1, "eps")]
    for rows, dim, eps, status, text in bad:
        with pytest.raises(isk.IskError) as e:
            isk.rmsnorm(A, A, A, rows, dim, eps, 0)
        assert e.value.status == status and text in e.value.message, (e.value.status, e.value.message)
    with pytest.raises(isk.IskError) as e:
        isk.rmsnorm(A + 8, A, A, 4, 64, 1e-6, 0)
    assert e.value.status == -1 and "aligned" in e.value.message
    isk.rmsnorm(None, None, None, 0, 64, 1e-6, 0)          # no rows: nothing to do


def test_linear_arguments_are_checked_before_any_device_work():
    A = 1 << 20
    bad = [(-1, 64, 128, -1, "m must"), (4, 24, 128, -2, "multiple of 16"), (4, 0, 128, -2, "multiple of 16"),
           (4, 64, 96, -2, "multiple of 128"), (4, 64, 0, -2, "multiple of 128")]
    for m, n, k, status, text in bad:
        with pytest.raises(isk.IskError) as e:
            isk.linear_bf16(A, A, A, m, n, k, 0)
        assert e.value.status == status and text in e.value.message, (e.value.status, e.value.message)
    with pytest.raises(isk.IskError) as e:
        isk.linear_bf16(A + 4, A, A, 4, 64, 128, 0)
    assert e.value.status == -1 and "aligned" in e.value.message
    isk.linear_bf16(None, None, None, 0, 64, 128, 0)      # no rows: nothing to do


# ----------------------------------------------------------------------------
# Length-band split tables (isk_plan_create_banded).

def band_rule(bands, U):
    """Split length of a row with U units, written from the band definition:
    the first band whose bound covers U (the last takes longer rows), and a
    split cap that stretches the splits to the next multiple of 64."""
    k = 0
    while k + 1 < len(bands) and U > bands[k][0]:
        k += 1
    _, S, cap = (tuple(bands[k]) + (0,))[:3]
    n = -(-U // S)
    if cap == 0 or n <= cap:
        return S
    per = -(-U // cap)
    return -(-per // 64) * 64


def banded_segments(desc, bands, lens, topk=None):
    with isk.Plan(desc, lens, topk, bands=bands) as p:
        return p.segments(), p.info()


BAND_TABLES = [
    [(1 << 30, 1536)],
    [(4096, 512), (32768, 1536), (1 << 30, 4096)],
    [(8192, 1024, 4), (65536, 2048, 16), (1 << 30, 1536, 24)],
    [(0, 64), (100, 128, 1), (2000, 192)],
]


@settings(max_examples=60, deadline=None)
@given(lens=st.lists(st.integers(0, 131072), min_size=1, max_size=20), table=st.sampled_from(range(len(BAND_TABLES))))
def test_banded_plan_follows_the_band_rule(lens, table):
    bands = BAND_TABLES[table]
    segs, info = banded_segments(mla_desc(max_pages_per_row=2048), bands, lens)
    _check_tiling(segs, info, lens, None)
    used = 0
    for r, U in enumerate(lens):
        mine = sorted((int(b), int(e)) for rr, b, e, _, _ in segs if rr == r)
        if U == 0:
            assert mine == []
            continue
        S = band_rule(bands, U)
        used = max(used, S)
        assert mine == [(i * S, min((i + 1) * S, U)) for i in range(-(-U // S))]
        cap = (tuple(bands[min(k for k in range(len(bands)) if U <= bands[k][0] or k == len(bands) - 1)]) + (0,))[2]
        assert cap == 0 or len(mine) <= cap
    assert info["split_tokens"] == used


def test_band_rule_examples():
    """Hand-worked values of the rule (a pin independent of the loop above)."""
    bands = [(8192, 1024, 4), (65536, 2048, 16), (1 << 30, 1536, 24)]
    assert band_rule(bands, 4096) == 1024          # 4 splits, at the cap
    assert band_rule(bands, 4097) == 1088          # 5 > 4: ceil(4097/4) = 1025 -> 1088
    assert band_rule(bands, 8192) == 2048          # ceil(8192/4) = 2048
    assert band_rule(bands, 8193) == 2048          # second band, 5 splits
    assert band_rule(bands, 65536) == 4096         # 32 > 16 splits: 65536/16
    assert band_rule(bands, 65537) == 2752         # third band: 43 > 24, ceil(65537/24) = 2731 -> 2752
    segs, _ = banded_segments(mla_desc(max_pages_per_row=2048), bands, [4097, 65537])
    r0 = sorted((int(b), int(e)) for r, b, e, _, _ in segs if r == 0)
    assert r0 == [(0, 1088), (1088, 2176), (2176, 3264), (3264, 4097)]
    assert sum(1 for r, *_ in segs if r == 1) == 24


def test_one_uncapped_band_plans_like_a_single_split_length():
    lens = [0, 1, 100, 1536, 1537, 40000, 131072]
    for S in (64, 512, 1536, 4096):
        a, ia = segments(mla_desc(max_pages_per_row=2048, split_tokens=S), lens)
        b, ib = banded_segments(mla_desc(max_pages_per_row=2048), [(1 << 30, S)], lens)
        assert np.array_equal(a, b) and ia == ib


@settings(max_examples=40, deadline=None)
@given(lens=st.lists(st.integers(0, 100000), min_size=1, max_size=24), probe=st.integers(0, 100000),
       pos=st.integers(0, 24), table=st.sampled_from(range(len(BAND_TABLES))))
def test_banded_splits_do_not_depend_on_batchmates(lens, probe, pos, table):
    desc, bands = mla_desc(max_pages_per_row=2048), BAND_TABLES[table]
    solo, _ = banded_segments(desc, bands, [probe])
    pos = min(pos, len(lens))
    batch = lens[:pos] + [probe] + lens[pos:]
    segs, _ = banded_segments(desc, bands, batch)
    assert sorted((b, e) for r, b, e, _, _ in segs if r == pos) == sorted((b, e) for _, b, e, _, _ in solo)


def test_banded_sparse_plan_uses_topk_len_and_update_keeps_the_table():
    bands = [(1024, 256), (1 << 30, 1024, 2)]
    desc = mla_desc(topk_width=4096, max_pages_per_row=2048)
    with isk.Plan(desc, [9000, 9000, 9000], [1000, 4096, 3000], bands=bands) as p:
        segs = p.segments()
        assert sorted((int(b), int(e)) for r, b, e, _, _ in segs if r == 0) == [(0, 256), (256, 512), (512, 768), (768, 1000)]
        assert sorted((int(b), int(e)) for r, b, e, _, _ in segs if r == 1) == [(0, 2048), (2048, 4096)]
        assert sorted((int(b), int(e)) for r, b, e, _, _ in segs if r == 2) == [(0, 1536), (1536, 3000)]
        p.update([10, 10], [300, 4096])
        segs = p.segments()
        assert sorted((int(b), int(e)) for r, b, e, _, _ in segs if r == 0) == [(0, 256), (256, 300)]
        assert sorted((int(b), int(e)) for r, b, e, _, _ in segs if r == 1) == [(0, 2048), (2048, 4096)]
        assert p.info()["split_tokens"] == 2048


def test_band_table_arguments_are_checked():
    lens = [100]
    cases = [
        (mla_desc(), [], "n_bands"),
        (mla_desc(), [(1 << 20 + k, 64) for k in range(17)], "n_bands"),
        (mla_desc(), [(100, 100)], "multiple of 64"),
        (mla_desc(), [(100, 0)], "multiple of 64"),
        (mla_desc(), [(100, 64, -1)], "max_splits"),
        (mla_desc(), [(100, 64), (100, 128)], "increasing"),
        (mla_desc(), [(-1, 64)], "increasing"),
        (mla_desc(split_tokens=512), [(100, 64)], "split_tokens"),
        (mla_desc(split_mode=isk.SPLIT_BATCH_BALANCED), [(100, 64)], "ISK_SPLIT_PER_ROW"),
    ]
    for desc, bands, needle in cases:
        with pytest.raises(isk.IskError) as ei:
            if bands:
                isk.plan_create_banded(desc, bands, lens)
            else:
                arr = isk.split_bands([(100, 64)])
                out = isk.ctypes.c_void_p()
                rc = isk.lib.isk_plan_create_banded(isk.ctypes.byref(desc), arr, 0, 1, isk._i32p(isk._i32_host(lens)),
                                                    None, isk.ctypes.byref(out))
                isk._check(rc)
        assert ei.value.status == -1 and needle in ei.value.message, (needle, ei.value.message)
    arr = isk.split_bands([(100, 64)])
    arr[0].reserved = 3
    with pytest.raises(isk.IskError, match="reserved"):
        isk.plan_create_banded(mla_desc(), arr, lens)
    out = isk.ctypes.c_void_p()
    assert isk.lib.isk_plan_create_banded(isk.ctypes.byref(mla_desc()), None, 1, 1,
                                          isk._i32p(isk._i32_host(lens)), None, isk.ctypes.byref(out)) == -1


# ----------------------------------------------------------------------------
# Split-kernel family of a plan
# ----------------------------------------------------------------------------

def test_split_kernel_family_follows_kind_heads_and_sparse_limits():
    """GQA and 64-head MLA have one family each; 128-head MLA runs the
    generated tile loop for dense rows and for sparse rows whose splits hold
    at most 1024 slots of pools of at most 4 GiB, the gather kernel for other
    sparse plans (a longer split, a larger main or extra pool)."""
    lens, tl = [5000, 3000], [2048, 700]
    fam = lambda desc, topk=None, **kw: isk.Plan(desc, lens, topk, **kw).info()["split_kernel"]
    # 50000 pages of 64 rows: a 3.7 GB pool (the default descriptor's 100000 pages exceed 4 GiB)
    sp = lambda **kw: mla_desc(topk_width=2048, num_pages=50000, **kw)
    assert fam(gqa_desc()) == isk.KERNEL_GQA
    assert fam(mla_desc(num_q_heads=64)) == isk.KERNEL_MLA_H16
    assert fam(mla_desc(num_q_heads=64, topk_width=2048), tl) == isk.KERNEL_MLA_H16
    assert fam(mla_desc()) == isk.KERNEL_MLA_H128
    assert fam(mla_desc(num_q_heads=256)) == isk.KERNEL_MLA_H128
    assert fam(sp(), tl) == isk.KERNEL_MLA_H128                                       # 512-slot splits
    assert fam(sp(split_tokens=1024), tl) == isk.KERNEL_MLA_H128
    assert fam(sp(split_tokens=1088), tl) == isk.KERNEL_MLA_H32
    rows_4g = (1 << 32) // 1152                                    # pool rows within 4 GiB
    assert fam(mla_desc(topk_width=2048), tl) == isk.KERNEL_MLA_H32                   # 7.4 GB pool
    assert fam(mla_desc(topk_width=2048, page_size=1, num_pages=rows_4g, max_pages_per_row=8192), tl) == \
        isk.KERNEL_MLA_H128
    assert fam(mla_desc(topk_width=2048, page_size=1, num_pages=rows_4g + 1, max_pages_per_row=8192), tl) == \
        isk.KERNEL_MLA_H32
    ok_x, big_x = xdesc(), xdesc(page_size=64, num_pages=rows_4g // 64 + 1)
    assert fam(sp(), tl, extra=ok_x, extra_topk_len_host=[100, 900]) == isk.KERNEL_MLA_H128
    assert fam(sp(), tl, extra=big_x, extra_topk_len_host=[100, 900]) == isk.KERNEL_MLA_H32
    # balanced mode: splits of this batch stay within 1024 slots
    assert fam(sp(split_mode=isk.SPLIT_BATCH_BALANCED), tl) == isk.KERNEL_MLA_H128
