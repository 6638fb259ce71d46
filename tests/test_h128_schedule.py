"""The schedule checker of the generated dense MLA tile loop (CPU only).

The generated loop passes the checker; and the checker is pinned by planted
mistakes of the kinds a hand schedule can make -- a dropped LDS wait, a
dropped barrier, a dropped vector-memory wait, a conversion left out, a V^T
read moved ahead of its address set-up (the ordering that once made tiles
1.. of a split use the previous tile's V) -- each of which it must report.
"""

import os
import sys

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "invariant_split_kv_amd", "csrc")
sys.path.insert(0, CSRC)
import check_mla_h128 as chk  # noqa: E402
import gen_mla_h128 as gen  # noqa: E402

SHORT = [(200, 0, 64), (97, 0, 64)]


@pytest.fixture(scope="module")
def lines():
    return gen.generate().split("\n")


def _index(lines, pred, start=0):
    return next(i for i in range(start, len(lines)) if pred(lines[i].strip()))


def test_generated_loop_passes():
    assert chk.check() == []


def test_window_reload_and_offset_split_are_walked():
    body = gen.generate()
    for n, begin, page in ((4200, 0, 64), (9000, 1536, 128), (300, 1600, 128)):
        w = chk._Wave(body.split("\n"), dict(ntiles=(n + 31) // 32, begin=begin, end=begin + n, P=page,
                                             npg=1 << 20, pbase=begin // page, on0=begin % page,
                                             pend=(begin + n + page - 1) // page, lds=0, w=2, kv_lo=0, kv_hi=0),
                      lambda s: False)
        loads = []
        step = w.step

        def counting(i, line, step=step):
            if line.startswith("global_load_dword "):
                loads.append(i)
            return step(i, line)

        w.step = counting
        assert w.run() == []
        pages = (begin + n + page - 1) // page - begin // page
        assert len(loads) == 1 + (pages - 1) // 64, (n, begin, page, len(loads))


def _drop(lines, i):
    return "\n".join(lines[:i] + lines[i + 1:])


def test_dropped_lds_wait_is_reported(lines):
    pv = _index(lines, lambda l: l.startswith("norescale_MA"))
    waits = [i for i in range(pv, pv + 400) if "lgkmcnt" in lines[i]]
    assert chk.check(_drop(lines, waits[1]), SHORT)


def test_dropped_barrier_is_reported(lines):
    ma = _index(lines, lambda l: l.startswith("MA_%="))
    assert chk.check(_drop(lines, _index(lines, lambda l: l == "s_barrier", ma)), SHORT)


def test_dropped_vector_memory_wait_is_reported(lines):
    mb = _index(lines, lambda l: l.startswith("MB_%="))
    assert chk.check(_drop(lines, _index(lines, lambda l: l.startswith("s_waitcnt vmcnt"), mb)), SHORT)


def test_dropped_conversion_is_reported(lines):
    pv = _index(lines, lambda l: l.startswith("norescale_MA"))
    assert chk.check(_drop(lines, _index(lines, lambda l: l.startswith("v_cvt_pkrtz_f16_f32"), pv)), SHORT)


def test_v_read_before_its_address_is_reported(lines):
    # move the V^T address set-up of the next tile after the first V^T read
    # that uses it
    pv = _index(lines, lambda l: l.startswith("norescale_MA"))
    a = _index(lines, lambda l: l.startswith("v_add_u32 v235,"), pv)
    r = _index(lines, lambda l: l.startswith("ds_read_b64_tr_b16") and "v235" in l, a)
    moved = lines[:a] + lines[a + 4:r + 1] + lines[a:a + 4] + lines[r + 1:]
    errs = chk.check("\n".join(moved), SHORT)
    assert any("V operand" in e for e in errs)


def test_scalar_load_check_of_the_gather_kernel_loop():
    """The build refuses scalar loads inside a kernel's inner (tile) loop; the
    check sees a planted one there and none in the segment loop around it."""
    sys.path.insert(0, os.path.dirname(CSRC))
    import build
    text = "\n".join([
        "kern:", "\ts_load_dword s4, s[0:1], 0x0",
        ".LBB0_1:                               ; =>This Loop Header: Depth=1",
        "\ts_load_dword s5, s[0:1], 0x4",
        ".LBB0_2:                               ;   Parent Loop BB0_1 Depth=1",
        "                                        ; =>  This Inner Loop Header: Depth=2",
        "\tv_mov_b32 v0, 0",
        "\ts_cbranch_scc1 .LBB0_2",
        ".LBB0_3:                               ;   in Loop: Header=BB0_1 Depth=1",
        "\ts_load_dword s6, s[0:1], 0x8",
    ])
    assert build.check_no_scalar_loads_in_tile_loop(text) == []
    planted = text.replace("\tv_mov_b32 v0, 0", "\ts_load_dword s7, s[0:1], 0xc")
    assert [s for _, s in build.check_no_scalar_loads_in_tile_loop(planted)] == ["s_load_dword s7, s[0:1], 0xc"]


# ----------------------------------------------------------------------------
# Sparse body: window-based tile loads and row-valid masks
# ----------------------------------------------------------------------------

SPARSE_SHORT = [(65, 0, 64), (300, 0, 64)]


@pytest.fixture(scope="module")
def sparse_body():
    return gen.generate(sparse=True)


def test_generated_sparse_loop_passes(sparse_body):
    assert chk.check(sparse_body, chk.SPARSE_SEGMENTS, sparse=True) == []


def test_sparse_load_with_the_wrong_piece_offset_is_reported(sparse_body):
    # a load adds the piece offset of another load to its window value
    old = f"v_add_u32_sdwa v146, v146, {gen.LO(6)} "
    assert old in sparse_body
    errs = chk.check(sparse_body.replace(old, f"v_add_u32_sdwa v146, v146, {gen.LO(5)} ", 1), SPARSE_SHORT,
                     sparse=True)
    assert any("piece offset" in e for e in errs)


def test_sparse_window_of_the_wrong_tile_is_reported(sparse_body):
    # window values read at 64 bytes a tile instead of 128
    old = f"s_lshl_b32 {gen.S_WINU}, {gen.S_LI}, 7"
    assert old in sparse_body
    errs = chk.check(sparse_body.replace(old, f"s_lshl_b32 {gen.S_WINU}, {gen.S_LI}, 6"), SPARSE_SHORT, sparse=True)
    assert any("reads the window of tile" in e for e in errs)


def test_sparse_mask_of_the_wrong_tile_is_reported(sparse_body):
    # scores of tile it+1 masked with tile it+2's mask
    old = f"v_lshrrev_b32_e64 {gen.T0}, {gen.T0}, {gen.S_NV1}"
    assert old in sparse_body
    errs = chk.check(sparse_body.replace(old, f"v_lshrrev_b32_e64 {gen.T0}, {gen.T0}, {gen.S_NV2}", 1),
                     SPARSE_SHORT, sparse=True)
    assert any("mask in" in e for e in errs)


def test_sparse_clobbered_tile0_mask_is_reported(sparse_body):
    # a scalar temporary that shares tile 0's mask register written in the
    # prologue before the mask is used (the kind of slip a prologue edit makes)
    lines = sparse_body.split("\n")
    z = _index(lines, lambda l: l.startswith("zskip_pro") or l.startswith(f"s_cmp_eq_u32 {gen.S_NV0}, -1"))
    planted = lines[:z] + [f"\ts_sub_u32 {gen.S_T3}, %[ntiles], 1"] + lines[z:]
    errs = chk.check("\n".join(planted), SPARSE_SHORT, sparse=True)
    assert any(f"mask in {gen.S_NV0}" in e for e in errs)
