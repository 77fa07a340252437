"""Pins of the overlapped two-stream compressor (oracle.csa.compress_c4a): closed forms,
reductions to the single-stream compressor, the overlap structure and chunking."""
import math

import numpy as np

from oracle import csa


def _rand(seed, T=16, d=5, m=4, lead=()):
    g = np.random.default_rng(seed)
    sh = lead + (T, d)
    return (g.standard_normal(sh), g.standard_normal(sh), g.standard_normal(sh),
            g.standard_normal(sh), 0.3 * g.standard_normal((m, d)), 0.3 * g.standard_normal((m, d)))


def test_hand_worked_m1():
    # m = 1, one channel: entry 0 is xa[0] alone (no previous block); entry 1 mixes xa[1]
    # (logit za[1] + ba = ln 3) and xb[0] (logit zb[0] + bb = 0): weights 3/4 and 1/4
    xa = np.array([[2.0], [4.0]]); za = np.array([[0.7], [math.log(3.0) - 0.5]])
    xb = np.array([[8.0], [100.0]]); zb = np.array([[-0.25], [9.0]])
    ba = np.array([[0.5]]); bb = np.array([[0.25]])
    out = csa.compress_c4a(xa, za, xb, zb, ba, bb, 1)
    assert np.allclose(out[:, 0], [2.0, 0.75 * 4.0 + 0.25 * 8.0], rtol=1e-15)


def test_uniform_logits_give_the_mean_of_the_eight_rows():
    xa, _, xb, _, _, _ = _rand(1)
    z = np.zeros_like(xa); b = np.zeros((4, 5))
    out = csa.compress_c4a(xa, z, xb, z, b, b, 4)
    assert np.allclose(out[0], xa[0:4].mean(axis=0))                  # entry 0: its own block
    for e in range(1, 4):
        want = (xa[4 * e:4 * e + 4].sum(axis=0) + xb[4 * e - 4:4 * e].sum(axis=0)) / 8
        assert np.allclose(out[e], want)


def test_masked_b_stream_is_the_single_stream_compressor():
    xa, za, xb, zb, ba, bb = _rand(2)
    out = csa.compress_c4a(xa, za, xb, zb - 1e4, ba, bb, 4)
    assert np.allclose(out, csa.compress(xa, za, ba, 4), rtol=1e-12, atol=1e-12)


def test_masked_a_stream_is_the_previous_block_of_b():
    xa, za, xb, zb, ba, bb = _rand(3)
    out = csa.compress_c4a(xa, za - 1e4, xb, zb, ba, bb, 4)
    assert np.allclose(out[1:], csa.compress(xb[:-4], zb[:-4], bb, 4), rtol=1e-12, atol=1e-12)


def test_every_token_feeds_exactly_two_entries():
    xa, za, xb, zb, ba, bb = _rand(4)
    base = csa.compress_c4a(xa, za, xb, zb, ba, bb, 4)
    t = 6                                          # block 1, so a-part of entry 1, b-part of 2
    for which in ("a", "b"):
        x2, z2 = (xa.copy(), za.copy()) if which == "a" else (xb.copy(), zb.copy())
        x2[t] += 1.0
        z2[t] += 0.5
        args = (x2, z2, xb, zb) if which == "a" else (xa, za, x2, z2)
        out = csa.compress_c4a(*args, ba, bb, 4)
        changed = np.flatnonzero(np.abs(out - base).max(axis=1) > 0)
        assert changed.tolist() == ([1] if which == "a" else [2])


def test_chunks_with_the_previous_block_equal_the_whole():
    xa, za, xb, zb, ba, bb = _rand(5, T=24, lead=(2,))
    whole = csa.compress_c4a(xa, za, xb, zb, ba, bb, 4)
    first = csa.compress_c4a(xa[:, :8], za[:, :8], xb[:, :8], zb[:, :8], ba, bb, 4)
    rest = csa.compress_c4a(xa[:, 8:], za[:, 8:], xb[:, 8:], zb[:, 8:], ba, bb, 4,
                            Xb_prev=xb[:, 4:8], Zb_prev=zb[:, 4:8])
    assert np.allclose(np.concatenate([first, rest], axis=1), whole, rtol=1e-14, atol=1e-14)


def test_weights_sum_to_one_and_stay_inside_the_rows():
    # a convex combination: every channel of an entry lies within its 2m rows' range
    xa, za, xb, zb, ba, bb = _rand(6, T=32)
    za *= 5; zb *= 5
    out = csa.compress_c4a(xa, za, xb, zb, ba, bb, 4)
    for e in range(1, 8):
        rows = np.concatenate([xa[4 * e:4 * e + 4], xb[4 * e - 4:4 * e]])
        assert np.all(out[e] <= rows.max(axis=0) + 1e-12)
        assert np.all(out[e] >= rows.min(axis=0) - 1e-12)
    ones = csa.compress_c4a(np.ones_like(xa), za, np.ones_like(xb), zb, ba, bb, 4)
    assert np.allclose(ones, 1.0, rtol=1e-14)
