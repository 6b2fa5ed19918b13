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


# ---- per-channel logits -----------------------------------------------------

def _brute_channel(x, Z, b, w, s):
    """Loops only: every entry, channel and window row, with math.exp."""
    import math
    L, C = len(x), len(x[0])
    N = (L - w) // s + 1 if L >= w else 0
    out = []
    for i in range(N):
        row = []
        for c in range(C):
            a = [Z[i * s + j][c] + b[j] for j in range(w)]
            mx = max(a)
            e = [math.exp(v - mx) for v in a]
            den = sum(e)
            row.append(sum(e[j] / den * x[i * s + j][c] for j in range(w)))
        out.append(row)
    return np.array(out)


@pytest.mark.parametrize("w,s", [(8, 4), (3, 2), (5, 5), (1, 1)])
def test_channel_logits_brute_force(w, s):
    L, C = 23, 4
    x = rng.standard_normal((L, C))
    Z = rng.standard_normal((L, C))
    b = rng.standard_normal(w) * 0.1
    np.testing.assert_allclose(oracle.compress_channel_logits(x, Z, b, w, s), _brute_channel(x, Z, b, w, s),
                               rtol=1e-13, atol=1e-14)


def test_channel_logits_reduce_to_per_token_and_mean():
    L, C, w, s = 40, 6, 8, 4
    x = rng.standard_normal((L, C))
    z = rng.standard_normal(L)
    b = rng.standard_normal(w) * 0.1
    # the same logit in every channel is the per-token form
    np.testing.assert_allclose(oracle.compress_channel_logits(x, np.repeat(z[:, None], C, 1), b, w, s),
                               oracle.compress(x, z, b, w, s), rtol=1e-13, atol=1e-14)
    # constant logits (any per-channel constants) and no bias: window means
    Zc = np.tile(rng.standard_normal(C), (L, 1))
    y = oracle.compress_channel_logits(x, Zc, None, w, s)
    for i in range(oracle.n_entries(L, w, s)):
        np.testing.assert_allclose(y[i], x[i * s:i * s + w].mean(0), rtol=1e-13, atol=1e-13)


def test_channel_logits_channels_are_independent_and_shift_invariant():
    L, C, w, s = 37, 5, 8, 4
    x = rng.standard_normal((L, C))
    Z = rng.standard_normal((L, C))
    b = rng.standard_normal(w) * 0.1
    y = oracle.compress_channel_logits(x, Z, b, w, s)
    # changing channel 3's values and logits leaves the other channels alone
    x2, Z2 = x.copy(), Z.copy()
    x2[:, 3] = rng.standard_normal(L)
    Z2[:, 3] = rng.standard_normal(L) * 5
    y2 = oracle.compress_channel_logits(x2, Z2, b, w, s)
    keep = [0, 1, 2, 4]
    np.testing.assert_array_equal(y2[:, keep], y[:, keep])
    assert not np.allclose(y2[:, 3], y[:, 3])
    # adding a constant to one channel's logits changes nothing
    Z3 = Z.copy()
    Z3[:, 1] += 7.0
    np.testing.assert_allclose(oracle.compress_channel_logits(x, Z3, b, w, s), y, rtol=1e-12, atol=1e-13)


def test_channel_logits_one_hot_picks_the_row():
    # a dominant logit at window row j of channel c returns x[i*s + j][c]
    # (exp(-60) ~ 1e-26 of weight on every other row)
    L, C, w, s = 32, 3, 8, 4
    x = rng.standard_normal((L, C))
    j_of_c = [0, 5, 7]
    for i in range(oracle.n_entries(L, w, s)):
        Zi = np.zeros((L, C))
        for c, j in enumerate(j_of_c):
            Zi[i * s + j, c] = 60.0
        y = oracle.compress_channel_logits(x, Zi, None, w, s)
        for c, j in enumerate(j_of_c):
            assert abs(y[i, c] - x[i * s + j, c]) < 1e-12


def test_index_keys_use_the_entries_own_weights():
    # K_I of an entry is the merge of its window's raw indexer keys with the
    # same softmax weights as its K|V: a dominant logit on window row j makes
    # both the entry and its indexer key the row j ones
    L, C, DI, w, s = 48, 8, 4, 8, 4
    x = rng.standard_normal((L, C))
    xi = rng.integers(-4, 5, (L, DI)).astype(float)
    z = np.zeros(L)
    z[4 * 3 + 6] = 80.0  # entry 3, window row 6 (also row 2 of entry 4)
    ckv, ki = oracle.compress_with_index(x, xi, z, None, w, s)
    np.testing.assert_allclose(ckv[3], x[18], atol=1e-12)
    np.testing.assert_allclose(ki[3], xi[18], atol=1e-12)
    np.testing.assert_allclose(ki[4], xi[18], atol=1e-12)
    # uniform logits: the indexer keys are window means of the raw keys
    _, ki0 = oracle.compress_with_index(x, xi, None, None, w, s)
    for i in range(oracle.n_entries(L, w, s)):
        np.testing.assert_allclose(ki0[i], xi[i * s:i * s + w].mean(0), rtol=1e-13, atol=1e-13)
