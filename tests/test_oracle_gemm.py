"""Pins of the matmul oracle: a pure-Python triple loop on small inputs,
integer inputs whose products and sums are exact, and the roles of the two
operands (a transposed or swapped operand fails)."""

import numpy as np
import pytest

import oracle


def loops(x, w):
    M, K = len(x), len(x[0])
    N = len(w)
    return np.array([[sum(float(x[m][k]) * float(w[n][k]) for k in range(K)) for n in range(N)] for m in range(M)])


def _pins(fn):
    rng = np.random.default_rng(9)
    res = []
    x = rng.standard_normal((3, 7))
    w = rng.standard_normal((5, 7))
    res.append(np.allclose(fn(x, w), loops(x, w), rtol=0, atol=1e-13))
    xi = rng.integers(-3, 4, (4, 64)).astype(np.float64)
    wi = rng.integers(-3, 4, (6, 64)).astype(np.float64)
    res.append(np.array_equal(fn(xi, wi), loops(xi, wi)))
    e = np.zeros((2, 4))
    e[0, 1] = 1.0
    e[1, 3] = 2.0
    w4 = np.arange(12, dtype=np.float64).reshape(3, 4)
    res.append(np.array_equal(fn(e, w4), np.array([[1.0, 5.0, 9.0], [6.0, 14.0, 22.0]])))
    return res


def test_oracle_passes_every_pin():
    assert all(_pins(oracle.linear))


@pytest.mark.parametrize("kind", ["dropped_last_k", "float32", "rows_reversed", "w_columns_reversed"])
def test_planted_mistakes_are_caught(kind):
    def fn(x, w):
        x, w = np.asarray(x, np.float64), np.asarray(w, np.float64)
        if kind == "dropped_last_k":
            return x[:, :-1] @ w[:, :-1].T
        if kind == "float32":
            return (x.astype(np.float32) @ w.astype(np.float32).T).astype(np.float64)
        if kind == "rows_reversed":
            return (x @ w.T)[::-1]
        return x @ w[:, ::-1].T
    assert not all(_pins(fn))
