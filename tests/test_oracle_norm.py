"""Pins of the RMSNorm oracle to things other than itself: torch's
rms_norm in float64 (a library routine), a 50-digit brute force, closed
forms, and planted mistakes that these pins must reject."""

import math

import numpy as np
import pytest

import oracle
from oracle import norm as on


def brute_force(x, w, eps, digits=50):
    import mpmath as mp
    mp.mp.dps = digits
    out = []
    for row in x:
        ms = mp.fsum(mp.mpf(float(v)) ** 2 for v in row) / len(row)
        r = 1 / mp.sqrt(ms + mp.mpf(float(eps)))
        out.append([float(mp.mpf(float(v)) * r * mp.mpf(float(wi))) for v, wi in zip(row, w)])
    return np.array(out)


def torch_rms_norm(x, w, eps):
    import torch
    t = torch.tensor(x, dtype=torch.float64)
    return torch.nn.functional.rms_norm(t, (t.shape[1],), weight=torch.tensor(w, dtype=torch.float64),
                                        eps=eps).numpy()


def _pins(fn):
    """All pins against the implementation `fn`; returns the list of results."""
    rng = np.random.default_rng(3)
    res = []
    x = rng.standard_normal((5, 48)) * 3.0
    w = rng.standard_normal(48)
    res.append(np.max(np.abs(fn(x, w, 1e-6) - torch_rms_norm(x, w, 1e-6))) < 1e-12)
    xs = rng.standard_normal((2, 7))
    ws = rng.standard_normal(7)
    res.append(np.max(np.abs(fn(xs, ws, 0.3) - brute_force(xs, ws, 0.3))) < 1e-13)
    c = np.full((1, 16), -2.5)
    res.append(np.allclose(fn(c, np.ones(16), 0.25), -2.5 / math.sqrt(6.25 + 0.25), atol=1e-15, rtol=0))
    y = fn(x, np.ones(48), 0.0)
    res.append(np.allclose(np.mean(y * y, axis=1), 1.0, atol=1e-13))
    res.append(np.allclose(fn(-7.0 * x, w, 0.0), -fn(x, w, 0.0), atol=1e-13))
    rows = np.stack([fn(x[r:r + 1], w, 1e-5)[0] for r in range(x.shape[0])])
    res.append(np.array_equal(rows, fn(x, w, 1e-5)))
    return res


def test_oracle_passes_every_pin():
    assert all(_pins(oracle.rmsnorm))


def _mutant(kind):
    def fn(x, w, eps):
        x = np.asarray(x, np.float64)
        w = np.asarray(w, np.float64)
        axis = 0 if kind == "wrong_axis" else 1
        s = np.sum(x * x, axis=axis, keepdims=True)
        ms = s if kind == "sum_not_mean" else s / x.shape[axis]
        if kind == "eps_outside_sqrt":
            d = np.sqrt(ms) + eps
        elif kind == "no_sqrt":
            d = ms + eps
        else:
            d = np.sqrt(ms + eps)
        y = x / d
        return y if kind == "no_weight" else y * w[None, :]
    return fn


@pytest.mark.parametrize("kind", ["wrong_axis", "sum_not_mean", "eps_outside_sqrt", "no_sqrt", "no_weight"])
def test_planted_mistakes_are_caught(kind):
    assert not all(_pins(_mutant(kind)))


def test_faithful_restatement_passes():
    assert all(_pins(_mutant("none")))
