"""Pins of the per-head RMSNorm and the partial RoPE (oracle.csa.rms_norm, oracle.csa.rope)."""
import math

import numpy as np

from oracle import csa


def test_rms_norm_hand_worked_and_invariants():
    x = np.array([3.0, -4.0, 0.0, 0.0])                   # mean square 25/4 -> rms 2.5
    g = np.array([1.0, 2.0, 1.0, 1.0])
    assert np.allclose(csa.rms_norm(x, g, eps=0.0), [1.2, -3.2, 0.0, 0.0], rtol=1e-15)
    r = np.random.default_rng(1).standard_normal((5, 64))
    ones = np.ones(64)
    y = csa.rms_norm(r, ones, eps=0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0)      # unit mean square
    assert np.allclose(csa.rms_norm(7.5 * r, ones, eps=0.0), y)   # scale invariant
    assert np.allclose(csa.rms_norm(r, ones), y, rtol=1e-5)       # eps is a small guard


def test_rope_hand_worked_pair():
    # rope_dim 2 on a 3-vector: only the last pair rotates, by pos * base^0 = pos radians
    x = np.array([5.0, 1.0, 0.0])
    y = csa.rope(x, 0.5, rope_dim=2)
    assert np.allclose(y, [5.0, math.cos(0.5), math.sin(0.5)], rtol=1e-15)
    # second pair of a rope_dim 4 part turns by pos * base^(-1/2)
    x = np.array([0.0, 0.0, 1.0, 0.0])
    y = csa.rope(x, 2.0, rope_dim=4, base=100.0)
    assert np.allclose(y, [0.0, 0.0, math.cos(0.2), math.sin(0.2)], rtol=1e-14)


def test_rope_is_a_rotation_of_the_last_dims_only():
    g = np.random.default_rng(2)
    x = g.standard_normal((3, 512))
    pos = np.array([0, 17, 1 << 20])
    y = csa.rope(x, pos)
    assert np.array_equal(y[:, :448], x[:, :448])
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))
    assert np.allclose(csa.rope(x, 0), x)
    assert np.allclose(csa.rope(y, -pos), x, atol=1e-12)            # inverse RoPE undoes it


def test_rope_scores_depend_on_the_distance_only():
    # <R(t) q, R(s) k> = <R(t - s) q, k> on the rotated part
    g = np.random.default_rng(3)
    q, k = g.standard_normal(64), g.standard_normal(64)
    for t, s in ((100, 40), (5000, 4940), (7, 7)):
        a = csa.rope(q, t) @ csa.rope(k, s)
        b = csa.rope(q, t - s) @ k
        assert math.isclose(a, b, rel_tol=1e-10, abs_tol=1e-10)
