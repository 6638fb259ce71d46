"""Length-band split tables (isk_plan_create_banded) on the GPU.

A band table makes a row's split length a piecewise function of its own
length (per-band split length and split cap), the form the FlashMLA issue page
"Sparse MLA decode is not batch-invariant ..." leaves open in its section
"Question".  The kernels see only the resulting segments, so these tests check
parity with the fp64 oracle on rows that land in every band (at the band
bounds, under and over each cap, with splits stretched to non-power-of-two
lengths), and that a one-band uncapped table gives the bits of the plain
per-row plan with the same split length.  Bit-level batch invariance under a
band table is checked in the invariance tests (config-5 stress batches).
"""

import math

import numpy as np
import pytest

from workloads import synth
from workloads.device import DeviceCase

from gpu_util import parity, reference

pytestmark = pytest.mark.gpu

# Band 0: short rows, 512-token splits.  Band 1: 1536-token splits, at most 6
# of them (rows above 9216 tokens get stretched splits).  Band 2: 4096-token
# splits, at most 12 (rows above 49152 tokens get stretched splits).
TABLE = [(2048, 512), (16384, 1536, 6), (1 << 30, 4096, 12)]
LENS = [0, 1, 65, 511, 2048, 2049, 9216, 9217, 16384, 16385, 49152, 60001]


def run(case, bands, **kw):
    print(f"[banded] {type(case).__name__} B={case.batch} bands={bands} kw={kw}", flush=True)
    dc = DeviceCase(case, bands=bands, **kw)
    dc.run()
    r = dc.result()
    dc.close()
    return r


@pytest.mark.parametrize("hq", [128, 16])
def test_mla_banded_parity(hq):
    case = synth.mla_case(LENS, hq, 1.0 / math.sqrt(192.0), 64, structure_seed=300 + hq)
    out, lse, _, _ = run(case, TABLE)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, f"mla banded hq={hq}")


def test_gqa_banded_parity():
    case = synth.gqa_case(LENS, 32, 8, 128, 1.0 / math.sqrt(128.0), 16, structure_seed=310)
    out, lse, _, _ = run(case, TABLE)
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, "gqa banded")


def test_sparse_banded_parity():
    lens = [0, 300, 700, 2048, 5000, 9000, 12000, 30000]
    case = synth.mla_case(lens, 128, 1.0 / math.sqrt(192.0), 64, structure_seed=320, topk_width=2048)
    out, lse, _, _ = run(case, [(256, 128), (1024, 256, 3), (1 << 30, 512, 2)])
    ro, rl = reference(case)
    parity(out, lse, ro, rl, False, "sparse banded")


def test_one_uncapped_band_gives_the_per_row_bits():
    case = synth.config3_mla(batch=16)
    _, _, bits, lbits = run(case, None)
    _, _, bbits, blbits = run(case, [(1 << 30, 1536)])
    assert np.array_equal(bits, bbits) and np.array_equal(lbits, blbits)
