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
    assert len(declared) == 11
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
    # longest splits are dispatched first
    lengths = segs[:, 2] - segs[:, 1]
    assert np.all(np.diff(lengths) <= 0)


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
        assert info["workspace_bytes"] >= expect * 128 * (512 + 1) * 4
        assert p.workspace_bytes == info["workspace_bytes"]
        p.update([100, 100])
        assert p.info()["num_partials"] == 0 and p.info()["batch"] == 2
