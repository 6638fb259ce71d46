"""Sparse 128-head MLA: the generated tile loop and the gather kernel give the
same bits.

Sparse plans whose splits hold at most 1024 top-k slots (of latent pools of
at most 4 GiB) run through the generated tile loop (mla_h128.hip), which
resolves a split's slots into an LDS window before its tile loads;
ISK_SPARSE_MLA_KERNEL=h32 routes them through the 32-head gather kernel
(mla_split_h32.hip) instead.  Both compute the same operations in the same
orders, so every output and LSE bit must agree.  The cases put masked slots
(-1 and positions at or past the length) at tile edges, fill whole tiles
with them, end splits on and next to tile edges, use small
pages, 1024-slot splits, 256 heads, an extra KV source and fp32 output.  The
gather kernel runs in a child process (the switch is read once per process);
both sides also stay within the oracle's bar, and each side's plan reports
the kernel family it ran.
"""

import json
import math
import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest

import invariant_split_kv_amd as isk
from workloads import synth
from workloads.device import DeviceCase

from gpu_util import parity, reference

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GARBAGE = int(synth.bf16_bits(np.array([3.0e4], np.float32))[0])   # unused pool slots: finite, large


def build(spec):
    """The synthetic case a spec names (the same in parent and child)."""
    kind = spec["kind"]
    rng = np.random.default_rng(spec["seed"] + 1)
    if kind == "extra":
        case = synth.mla_extra_case(spec["lens"], spec["xlens"], 128, 1.0 / math.sqrt(192.0), 64,
                                    structure_seed=spec["seed"], topk_width=spec["W"], extra_width=spec["XW"],
                                    extra_page_size=16, split_tokens=spec["split"])
        xr = case.extra.rows
        xr[1].topk_idx[[0, 31, 32, 95]] = -1
        xr[2].topk_idx[[3, 4]] = [10 ** 6, spec["xlens"][2]]
        return case
    case = synth.mla_case(spec["lens"], spec["hq"], 1.0 / math.sqrt(192.0), spec["page"],
                          structure_seed=spec["seed"], topk_width=spec["W"], split_tokens=spec["split"])
    rows = case.rows
    if kind == "edges":
        # topk_len on and next to tile and split edges
        for b, tl in enumerate(spec["topk_lens"]):
            rows[b].topk_len = min(tl, int(rows[b].topk_len))
        rows[0].topk_idx[[0, 31, 32, 63, 64, 511, 512]] = -1               # tile and split edges
        rows[1].topk_idx[[5, 6]] = [spec["lens"][1], 10 ** 7]               # at and past the length
        rows[2].topk_idx[64:96] = -1                                        # a whole tile masked
        rows[3].topk_idx[rng.integers(0, 600, 40)] = -1                     # scattered
    else:
        rows[0].topk_idx[[0, 1, 1023, 1024]] = -1
        rows[1].topk_idx[96:160] = -1                                       # two whole tiles
        rows[2].topk_idx[rng.integers(0, 2000, 100)] = -1
    return case


CASES = {
    "edges": dict(kind="edges", lens=[3000, 900, 2500, 700, 5000, 1, 33, 4000, 1200],
                  topk_lens=[1024, 900, 600, 700, 513, 1, 33, 31, 65], W=1024, hq=128, page=64, split=0, seed=400),
    "split1024_page16": dict(kind="big", lens=[9000, 4000, 6000, 2100], W=2048, hq=128, page=16, split=1024,
                             seed=401),
    "hq256_page8": dict(kind="big", lens=[5000, 3000, 2500], W=2048, hq=256, page=8, split=512, seed=402),
    "extra": dict(kind="extra", lens=[3000, 900, 4000], xlens=[600, 1500, 2000], W=700, XW=1100, split=0,
                  seed=403),
}

CHILD = r"""
import sys, json, numpy as np
sys.path.insert(0, {root!r}); sys.path.insert(0, {root!r} + "/tests")
from test_gpu_sparse_kernels import build, GARBAGE
from workloads.device import DeviceCase
spec = json.loads({spec!r})
case = build(spec)
for f32 in (0, 1):
    dc = DeviceCase(case, out_f32=bool(f32), fill=GARBAGE)
    fam = dc.plan.info()["split_kernel"]
    dc.run()
    _, _, bits, lbits = dc.result()
    dc.close()
    np.save({out!r} + f"/bits{{f32}}.npy", bits)
    np.save({out!r} + f"/lbits{{f32}}.npy", lbits)
print("child family", fam, flush=True)
"""


@pytest.mark.parametrize("name", list(CASES))
def test_generated_sparse_loop_matches_gather_kernel_bits(name):
    spec = CASES[name]
    print(f"[case] sparse kernels {name}", flush=True)
    case = build(spec)
    ro, rl = reference(case)
    mine = {}
    for f32 in (0, 1):
        dc = DeviceCase(case, out_f32=bool(f32), fill=GARBAGE)
        assert dc.plan.info()["split_kernel"] == isk.KERNEL_MLA_H128
        dc.run()
        out, lse, bits, lbits = dc.result()
        dc.close()
        parity(out, lse, ro, rl, bool(f32), f"generated sparse loop {name} f32={f32}")
        mine[f32] = (bits, lbits)
    with tempfile.TemporaryDirectory() as d:
        env = dict(os.environ, ISK_SPARSE_MLA_KERNEL="h32")
        code = CHILD.format(root=ROOT, spec=json.dumps(spec), out=d)
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
        assert f"child family {isk.KERNEL_MLA_H32}" in r.stdout, r.stdout[-500:]
        for f32 in (0, 1):
            bits = np.load(os.path.join(d, f"bits{f32}.npy"))
            lbits = np.load(os.path.join(d, f"lbits{f32}.npy"))
            if not (np.array_equal(bits, mine[f32][0]) and np.array_equal(lbits, mine[f32][1])):
                nd = int(np.sum(bits != mine[f32][0]))
                nl = int(np.sum(lbits != mine[f32][1]))
                pytest.fail(f"{name} f32={f32}: {nd} output and {nl} lse bit patterns differ between the kernels")
