"""The two dense 128-head MLA kernels give the same bits.

Dense MLA with a head count that is a multiple of 128 runs through the
generated tile loop (mla_h128.hip); ISK_DENSE_MLA_KERNEL=h32 routes it through
the gather kernel (mla_split_h32.hip) instead.  Both compute the same
operations in the same orders, so on the same inputs every output and LSE
bit must agree.  The second kernel runs in a child process (the switch is
read once per process); both sides also stay within the oracle's bar.
"""

import math
import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest

from workloads import synth
from workloads.device import DeviceCase

from gpu_util import parity, reference

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CASES = {
    "edges": dict(lens=[0, 1, 2, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1535, 1536, 1537, 3100], hq=128, page=64,
                  split=0, seed=300),
    "hq256_p128_s256": dict(lens=[3000, 129, 5000, 64, 1], hq=256, page=128, split=256, seed=301),
    "long_splits": dict(lens=[9000, 20000, 8192], hq=128, page=64, split=8192, seed=302),
}

CHILD = r"""
import sys, json, numpy as np
sys.path.insert(0, {root!r}); sys.path.insert(0, {root!r} + "/tests")
import math
from workloads import synth
from workloads.device import DeviceCase
c = json.loads({spec!r})
case = synth.mla_case(c["lens"], c["hq"], 1.0 / math.sqrt(192.0), c["page"], structure_seed=c["seed"],
                      split_tokens=c["split"])
for f32 in (0, 1):
    dc = DeviceCase(case, out_f32=bool(f32))
    dc.run()
    _, _, bits, lbits = dc.result()
    dc.close()
    np.save({out!r} + f"/bits{{f32}}.npy", bits)
    np.save({out!r} + f"/lbits{{f32}}.npy", lbits)
print("child done", flush=True)
"""


@pytest.mark.parametrize("name", list(CASES))
def test_generated_loop_matches_gather_kernel_bits(name):
    import json
    c = CASES[name]
    print(f"[case] dense kernels {name}: {c}", flush=True)
    case = synth.mla_case(c["lens"], c["hq"], 1.0 / math.sqrt(192.0), c["page"], structure_seed=c["seed"],
                          split_tokens=c["split"])
    ro, rl = reference(case)
    mine = {}
    for f32 in (0, 1):
        dc = DeviceCase(case, out_f32=bool(f32))
        dc.run()
        out, lse, bits, lbits = dc.result()
        dc.close()
        parity(out, lse, ro, rl, bool(f32), f"generated loop {name} f32={f32}")
        mine[f32] = (bits, lbits)
    with tempfile.TemporaryDirectory() as d:
        env = dict(os.environ, ISK_DENSE_MLA_KERNEL="h32")
        code = CHILD.format(root=ROOT, spec=json.dumps(c), out=d)
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
        for f32 in (0, 1):
            bits = np.load(os.path.join(d, f"bits{f32}.npy"))
            lbits = np.load(os.path.join(d, f"lbits{f32}.npy"))
            same = np.array_equal(bits, mine[f32][0]) and np.array_equal(lbits, mine[f32][1])
            if not same:
                nd = int(np.sum(bits != mine[f32][0]))
                nl = int(np.sum(lbits != mine[f32][1]))
                pytest.fail(f"{name} f32={f32}: {nd} output and {nl} lse bit patterns differ between the kernels")
