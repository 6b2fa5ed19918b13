"""Pins for the compression oracle (CPU)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def test_worked_examples():
    ex = json.load(open(os.path.join(GOLD, "worked_examples.json")))
    for key in ("compress", "compress_bias"):
        e = ex[key]
        y = oracle.compress(np.array(e["x"]), np.array(e["z"]), np.array(e["b"]), e["w"], e["s"])
        np.testing.assert_allclose(y, np.array(e["y"]), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("w,s", [(128, 128), (4, 4), (8, 8)])
def test_uniform_weights_disjoint_is_mean_pooling(w, s):
    L, C = 5 * w + 3, 6
    x = rng.standard_normal((L, C))
    N = oracle.n_entries(L, w, s)
    y = oracle.compress(x, None, None, w, s)
    ref = x[: N * w].reshape(N, w, C).mean(axis=1)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)
    # a constant logit per token and a constant bias are also uniform weights
    y2 = oracle.compress(x, np.full(L, 2.5), np.full(w, -1.0), w, s)
    np.testing.assert_allclose(y2, ref, rtol=1e-13, atol=1e-13)


def test_uniform_weights_overlapping_is_window_mean():
    L, C, w, s = 61, 5, 8, 4
    x = rng.standard_normal((L, C))
    y = oracle.compress(x, None, None, w, s)
    for i in range(oracle.n_entries(L, w, s)):
        np.testing.assert_allclose(y[i], x[i * s : i * s + w].mean(axis=0), rtol=1e-13, atol=1e-13)


def test_one_hot_logit_selects_that_token():
    # A logit far above the rest puts all weight on one raw token: catches an
    # off-by-one in which token a logit or a bias belongs to.
    L, C, w, s = 40, 3, 8, 4
    x = rng.standard_normal((L, C))
    for i in range(oracle.n_entries(L, w, s)):
        for j in (0, 3, 7):
            z = np.zeros(L)
            z[i * s + j] = 800.0
            y = oracle.compress(x, z, None, w, s)
            np.testing.assert_allclose(y[i], x[i * s + j], rtol=0, atol=1e-12)
    # the same with the bias: position j of every window wins
    for j in (0, 5, 7):
        b = np.zeros(w)
        b[j] = 800.0
        y = oracle.compress(x, None, b, w, s)
        for i in range(oracle.n_entries(L, w, s)):
            np.testing.assert_allclose(y[i], x[i * s + j], rtol=0, atol=1e-12)


def test_shift_invariance_constant_identity_bounds_linearity():
    L, C, w, s = 77, 4, 8, 4
    x = rng.standard_normal((L, C))
    x2 = rng.standard_normal((L, C))
    z = rng.standard_normal(L)
    b = 0.1 * rng.standard_normal(w)
    y = oracle.compress(x, z, b, w, s)
    np.testing.assert_allclose(oracle.compress(x, z + 3.0, b - 7.0, w, s), y, rtol=1e-12, atol=1e-12)
    c = rng.standard_normal(C)
    np.testing.assert_allclose(oracle.compress(np.tile(c, (L, 1)), z, b, w, s),
                               np.tile(c, (oracle.n_entries(L, w, s), 1)), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.compress(x, z, np.zeros(1), 1, 1), x, rtol=0, atol=0)
    for i in range(y.shape[0]):
        win = x[i * s : i * s + w]
        assert np.all(y[i] <= win.max(axis=0) + 1e-12) and np.all(y[i] >= win.min(axis=0) - 1e-12)
    np.testing.assert_allclose(oracle.compress(2 * x - 3 * x2, z, b, w, s),
                               2 * y - 3 * oracle.compress(x2, z, b, w, s), rtol=1e-11, atol=1e-11)


def test_no_complete_window():
    assert oracle.compress(np.ones((5, 2)), None, None, 8, 4).shape == (0, 2)
