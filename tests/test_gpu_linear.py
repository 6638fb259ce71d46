"""Batch-invariant linear layer (isk_linear_bf16) on the GPU: parity with the
fp64 oracle and bit equality of a row across row counts that cross the
tile-shape switches at 16, 32 and 64 rows.  Above 64 rows, with K a multiple of
256, tiles are the smallest of 128 x 64, 128 x 128 and 256 x 128 whose count
fits one round on 256 CUs (n = 4096: 300 rows take 128 x 64, 600 rows 128 x 128,
1100 rows 256 x 128); other K take 128 x 128 tiles with 32-wide K stages
(K = 640).

Bar: bf16 x bf16 products are exact in fp32, so the only errors are the
fp32 additions of the K products; whatever their order, the error of an
element is at most (K + 3) * 2^-24 * sum_k |x_k w_k| (K products plus three
partial sums).  Integer inputs whose sums stay below 2^24 must come out
exact.
"""

import numpy as np
import pytest
import torch

import invariant_split_kv_amd as isk
import oracle
from workloads import synth

pytestmark = pytest.mark.gpu


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def run(xbits, wbits):
    m, k = xbits.shape
    n = wbits.shape[0]
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    isk.linear_bf16(to_dev(xbits), to_dev(wbits), y, m, n, k)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def rows(m, k, seed, std=1.0):
    out = np.empty((m, k), np.uint16)
    for r in range(m):
        out[r] = synth.draw_bf16(np.random.default_rng([seed, r]), (k,), std)
    return out


@pytest.mark.parametrize("m", [1, 20, 33, 100, 300])
def test_integer_inputs_are_exact(m):
    rng = np.random.default_rng(m)
    k, n = 512, 64
    xb = synth.bf16_bits(rng.integers(-3, 4, (m, k)).astype(np.float32))
    wb = synth.bf16_bits(rng.integers(-3, 4, (n, k)).astype(np.float32))
    y = run(xb, wb)
    ref = oracle.linear(synth.bf16_value(xb), synth.bf16_value(wb))
    assert np.array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (16, 256, 4096), (17, 96, 2048), (32, 64, 1024), (33, 128, 4096),
                                   (256, 48, 512), (257, 48, 512), (64, 4096, 1024), (300, 256, 1024),
                                   (1000, 400, 4096), (300, 160, 640), (40, 48, 1024), (9, 80, 512), (600, 4096, 256), (1100, 4096, 256)])
def test_linear_parity(m, n, k):
    xb, wb = rows(m, k, 40 + m), rows(n, k, 41, std=0.05)
    y = run(xb, wb).astype(np.float64)
    xv, wv = synth.bf16_value(xb).astype(np.float64), synth.bf16_value(wb).astype(np.float64)
    ref = oracle.linear(xv, wv)
    bound = (k + 3) * 2.0 ** -24 * (np.abs(xv) @ np.abs(wv).T)
    err = np.abs(y - ref)
    print(f"[linear] m={m} n={n} k={k} max_abs={err.max():.3g} max_err/bound={np.max(err / bound):.3g}", flush=True)
    assert np.all(err <= bound)


@pytest.mark.parametrize("k", [640, 1024, 4096])
def test_row_bits_do_not_depend_on_the_row_count(k):
    n = 256
    wb = rows(n, k, 51, std=0.05)
    probe = rows(1, k, 52)[0]
    solo = run(probe[None, :], wb)[0]
    for m in (2, 16, 17, 31, 32, 33, 64, 65, 100, 256, 257, 1000):
        xb = rows(m, k, 53 + m)
        pos = (5 * m) // 7
        xb[pos] = probe
        y = run(xb, wb)
        assert np.array_equal(y[pos], solo), f"m={m}: probe row bits differ"


def test_row_bits_across_lds_tile_heights():
    """n = 4096: 300 rows take 128 x 64 tiles (3 x 64 = 192), 600 rows
    128 x 128 (5 x 64 = 320 tiles of 128 x 64 would not fit one round on 256
    CUs, 5 x 32 = 160 do), 1100 rows 256 x 128 (9 x 32 = 288 would not); a
    probe row's bits match its solo run."""
    n, k = 4096, 256
    wb = rows(n, k, 61, std=0.05)
    probe = rows(1, k, 62)[0]
    solo = run(probe[None, :], wb)[0]
    for m in (300, 600, 1100):
        xb = rows(m, k, 63 + m)
        pos = (3 * m) // 5
        xb[pos] = probe
        y = run(xb, wb)
        assert np.array_equal(y[pos], solo), f"m={m}: probe row bits differ"
