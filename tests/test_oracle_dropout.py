"""Pins of the dropout oracle (LoRA dropout on the low-rank branch's input).

Independent routes: with every element kept and p = 0 it is the layer of the C
oracle (oracle.forward / oracle.backward); its gradients match central finite
differences of the fp64 forward for a fixed mask; a dropped input column leaves
the low-rank branch untouched by that column."""
import numpy as np
import pytest

import oracle
from oracle import dropout


def _r(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _layer(M=6, N=5, K=8, r=3, seed=0):
    return (_r((M, K), seed), _r((N, K), seed + 1, 0.3), _r((r, K), seed + 2, 0.5), _r((N, r), seed + 3, 0.5),
            _r((M, N), seed + 4))


def test_no_dropout_is_the_layer():
    x, W, A, B, dY = (a.astype(np.float32) for a in _layer())
    ones = np.ones_like(x)
    np.testing.assert_allclose(dropout.forward(x, W, A, B, 1.5, ones, 0.0), oracle.forward(x, W, A, B, 1.5),
                               rtol=1e-12, atol=1e-12)
    for got, ref in zip(dropout.backward(x, W, A, B, dY, 1.5, ones, 0.0), oracle.backward(x, W, A, B, dY, 1.5)):
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("p", [0.1, 0.5])
def test_gradients_match_finite_differences(p):
    x, W, A, B, dY = _layer(seed=10)
    mask = (np.random.default_rng(11).random(x.shape) >= p).astype(np.float64)
    s, h = 2.0, 1e-6
    dX, dA, dB = dropout.backward(x, W, A, B, dY, s, mask, p)

    def L(x_, A_, B_):  # the scalar <dY, y>, whose gradients are the layer's
        return float(np.sum(dY * dropout.forward(x_, W, A_, B_, s, mask, p)))

    for name, arr, g in (("x", x, dX), ("A", A, dA), ("B", B, dB)):
        for idx in [(0, 0), (arr.shape[0] - 1, arr.shape[1] - 1), (1, 2)]:
            up, dn = arr.copy(), arr.copy()
            up[idx] += h
            dn[idx] -= h
            args_up = {"x": (up, A, B), "A": (x, up, B), "B": (x, A, up)}[name]
            args_dn = {"x": (dn, A, B), "A": (x, dn, B), "B": (x, A, dn)}[name]
            fd = (L(*args_up) - L(*args_dn)) / (2 * h)
            assert fd == pytest.approx(g[idx], rel=1e-6, abs=1e-9), (name, idx)


def test_dropped_column_does_not_reach_the_branch():
    x, W, A, B, _ = _layer(seed=20)
    mask = np.ones_like(x)
    mask[:, 3] = 0.0
    x2 = x.copy()
    x2[:, 3] += 5.0  # only the base path sees the change
    base_delta = (x2 - x) @ W.T
    y1 = dropout.forward(x, W, A, B, 1.0, mask, 0.25)
    y2 = dropout.forward(x2, W, A, B, 1.0, mask, 0.25)
    np.testing.assert_allclose(y2 - y1, base_delta, rtol=1e-12, atol=1e-12)
