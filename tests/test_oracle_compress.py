"""Pins of the oracle compressor (channel-wise softmax pooling with positional bias).

Each pin fails on a plausible mistake: a dropped bias, a transposed bias, a softmax over
channels instead of positions, a wrong entry/position index, a sign error."""
import numpy as np
import pytest
from scipy.special import expit, softmax

from oracle import csa
from golden_util import arr, load


def rnd(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


def test_hand_worked_example():
    g = load("hand_worked.json")["compress_m2"]
    out = csa.compress(arr(g["X"]), arr(g["Z"]), arr(g["bias"]), g["m"])
    np.testing.assert_allclose(out, arr(g["expected"]), rtol=0, atol=1e-14)


def test_uniform_logits_give_the_mean():
    # Z + bias constant over the pooled positions -> arithmetic mean of the rows
    m, d = 4, 16
    X = rnd(3, 8 * m, d, seed=1)
    bias = rnd(m, d, seed=2)
    Z = np.broadcast_to(5.0 - bias, (3, 8, m, d)).reshape(3, 8 * m, d)
    out = csa.compress(X, Z, bias, m)
    np.testing.assert_allclose(out, X.reshape(3, 8, m, d).mean(axis=2), rtol=0, atol=1e-14)


def test_m1_is_identity():
    X, Z = rnd(2, 9, 5, seed=3), rnd(2, 9, 5, seed=4)
    out = csa.compress(X, Z, rnd(1, 5, seed=5), 1)
    np.testing.assert_array_equal(out, X)


def test_m2_closed_form_sigmoid():
    # alpha_0 = sigma(a_0 - a_1) (scipy's logistic function)
    X, Z, b = rnd(10, 7, seed=6), rnd(10, 7, seed=7), rnd(2, 7, seed=8)
    out = csa.compress(X, Z, b, 2)
    a = Z.reshape(5, 2, 7) + b
    al0 = expit(a[:, 0] - a[:, 1])
    Xr = X.reshape(5, 2, 7)
    np.testing.assert_allclose(out, al0 * Xr[:, 0] + (1 - al0) * Xr[:, 1], rtol=1e-13, atol=1e-15)


def test_dominant_bias_position_copies_that_row():
    # a large bias at position j* of channel c copies row j* of every entry in channel c
    m, d = 4, 6
    X = rnd(16, d, seed=9)
    Z = rnd(16, d, seed=10)
    bias = np.zeros((m, d))
    jstar = [0, 1, 2, 3, 2, 1]
    for c, j in enumerate(jstar):
        bias[j, c] = 80.0
    out = csa.compress(X, Z, bias, m)
    Xr = X.reshape(4, m, d)
    for c, j in enumerate(jstar):
        np.testing.assert_allclose(out[:, c], Xr[:, j, c], rtol=1e-12)


def test_weights_sum_to_one_and_channels_independent():
    m, d = 3, 11
    Z, b = rnd(12, d, seed=11), rnd(m, d, seed=12)
    ones = csa.compress(np.ones((12, d)), Z, b, m)
    np.testing.assert_allclose(ones, 1.0, rtol=1e-14)
    X = rnd(12, d, seed=13)
    perm = np.random.default_rng(0).permutation(d)
    out = csa.compress(X, Z, b, m)
    outp = csa.compress(X[:, perm], Z[:, perm], b[:, perm], m)
    np.testing.assert_allclose(outp, out[:, perm], rtol=1e-14)


def test_library_softmax_over_positions():
    m, d = 4, 8
    X, Z, b = rnd(2, 12, d, seed=14), rnd(2, 12, d, seed=15), rnd(m, d, seed=16)
    P = softmax(Z.reshape(2, 3, m, d) + b, axis=2)
    ref = np.einsum("bemd,bemd->bed", P, X.reshape(2, 3, m, d))
    np.testing.assert_allclose(csa.compress(X, Z, b, m), ref, rtol=1e-13, atol=1e-15)


def test_entries_only_see_their_own_rows():
    m, d = 4, 5
    X, Z, b = rnd(20, d, seed=17), rnd(20, d, seed=18), rnd(m, d, seed=19)
    base = csa.compress(X, Z, b, m)
    X2 = X.copy()
    X2[8:12] += 100.0      # rows of entry 2 only
    out = csa.compress(X2, Z, b, m)
    np.testing.assert_array_equal(np.delete(out, 2, axis=0), np.delete(base, 2, axis=0))
    assert np.all(np.abs(out[2] - base[2]) > 1.0)


def test_extreme_logits_are_stable():
    m, d = 4, 3
    X = rnd(8, d, seed=20)
    Z = np.full((8, d), 700.0)
    Z[::4] = 800.0                 # exp overflow without the max shift
    out = csa.compress(X, Z, np.zeros((m, d)), m)
    np.testing.assert_allclose(out, X[::4], rtol=1e-12)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        csa.compress(np.zeros((6, 2)), np.zeros((6, 2)), np.zeros((4, 2)), 4)
    with pytest.raises(ValueError):
        csa.compress(np.zeros((8, 2)), np.zeros((8, 2)), np.zeros((2, 4)), 4)
