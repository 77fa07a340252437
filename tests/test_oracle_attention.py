"""Pins of the oracle's sparse attention with window and sink."""
import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle import csa, pipeline
from golden_util import arr, load


def rnd(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


def sdpa(q, rows, scale, sink=None):
    """torch's scaled_dot_product_attention in float64 (a library routine). The sink is an
    extra key with logit z'_h and a zero value: append a coordinate that is 1 in q, 0 in
    every row and z'_h/scale in the per-head sink key."""
    H, D = q.shape
    J = rows.shape[0]
    qq = torch.tensor(q)[None, :, None, :]                    # [1, H, 1, D]
    kk = torch.tensor(rows)[None, None].expand(1, H, J, D)
    vv = kk
    if sink is not None:
        qq = torch.cat([qq, torch.ones(1, H, 1, 1, dtype=torch.float64)], -1)
        kk = torch.cat([kk, torch.zeros(1, H, J, 1, dtype=torch.float64)], -1)
        ks = torch.zeros(1, H, 1, D + 1, dtype=torch.float64)
        ks[0, :, 0, D] = torch.tensor(sink) / scale
        kk = torch.cat([kk, ks], 2)
        vv = torch.cat([vv, torch.zeros(1, H, 1, D, dtype=torch.float64)], 2)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
    return o[0, :, 0, :].numpy()


def test_hand_worked():
    g = load("hand_worked.json")["attention"]
    kw = dict(w_cap=g["w_cap"], window=g["window"], t=g["t"], scale=g["scale"])
    o = pipeline.attend_row(arr(g["q"]), arr(g["kv"]), g["idx"], arr(g["ring"]), sink=arr(g["sink"]), **kw)
    np.testing.assert_allclose(o, arr(g["expected"]), rtol=1e-13)
    o2 = pipeline.attend_row(arr(g["q"]), arr(g["kv"]), g["idx"], arr(g["ring"]), sink=None, **kw)
    np.testing.assert_allclose(o2, arr(g["no_sink_expected"]), rtol=1e-13)


@pytest.mark.parametrize("seed", range(5))
def test_sink_attention_matches_library_sdpa(seed):
    H, D, J = 6, 24, 37
    q, rows, sink = rnd(H, D, seed=seed), rnd(J, D, seed=seed + 50), 2 * rnd(H, seed=seed + 99)
    sc = 1 / np.sqrt(D)
    np.testing.assert_allclose(csa.sink_attention(q, rows, sink, sc), sdpa(q, rows, sc, sink),
                               rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(csa.sink_attention(q, rows, None, sc), sdpa(q, rows, sc),
                               rtol=1e-11, atol=1e-13)


def test_sink_to_minus_infinity_is_plain_softmax_attention():
    q, rows = rnd(4, 8, seed=1), rnd(9, 8, seed=2)
    np.testing.assert_allclose(csa.sink_attention(q, rows, np.full(4, -1e300), 0.3),
                               sdpa(q, rows, 0.3), rtol=1e-12)


def test_single_row_closed_form():
    # one key, with sink: out = v * sigma(z - z')   (scipy's logistic function)
    q, v, sink = rnd(3, 5, seed=3), rnd(1, 5, seed=4), rnd(3, seed=5)
    z = 0.7 * (q @ v[0])
    np.testing.assert_allclose(csa.sink_attention(q, v, sink, 0.7),
                               expit(z - sink)[:, None] * v, rtol=1e-13)
    # without sink the single row is copied exactly
    np.testing.assert_allclose(csa.sink_attention(q, v, None, 0.7), np.repeat(v, 3, 0), rtol=1e-15)


def test_mass_below_one_with_sink():
    q, rows, sink = rnd(5, 8, seed=6), rnd(11, 8, seed=7), rnd(5, seed=8)
    q1 = np.hstack([q, np.zeros((5, 1))])
    rows1 = np.hstack([rows, np.ones((11, 1))])
    mass = csa.sink_attention(q1, rows1, sink, 0.5)[:, -1]
    # the constant-1 channel measures the attention mass; it equals 1 - sink weight
    lse = np.log(np.exp(0.5 * (q @ rows.T)).sum(1))
    np.testing.assert_allclose(mass, 1 - expit(sink - lse), rtol=1e-12)
    assert np.all(mass < 1)
    big = csa.sink_attention(q, rows, np.full(5, 60.0), 0.5)
    assert np.abs(big).max() < 1e-20       # a head can abstain almost entirely


def test_empty_rows_give_zero():
    assert np.all(csa.sink_attention(rnd(2, 4), np.zeros((0, 4)), None, 1.0) == 0)
    assert np.all(csa.sink_attention(rnd(2, 4), np.zeros((0, 4)), np.zeros(2), 1.0) == 0)


def test_permutation_of_selection_is_irrelevant():
    kv, ring = rnd(30, 8, seed=9), rnd(16, 8, seed=10)
    q, sink = rnd(3, 8, seed=11), rnd(3, seed=12)
    idx = np.array([4, 17, -1, 2, 29, 8])
    a = pipeline.attend_row(q, kv, idx, ring, 16, 5, 40, sink, 0.4)
    b = pipeline.attend_row(q, kv, idx[::-1], ring, 16, 5, 40, sink, 0.4)
    np.testing.assert_allclose(a, b, rtol=1e-13)


def test_window_range_and_ring_rows():
    # query t reads ring rows of positions [t-W+1, t] only, at row p % w_cap
    kv, q, sink = rnd(10, 6, seed=13), rnd(2, 6, seed=14), rnd(2, seed=15)
    ring = rnd(12, 6, seed=16)
    t, W, wc = 30, 5, 12
    base = pipeline.attend_row(q, kv, [1, 3], ring, wc, W, t, sink, 0.5)
    for p in range(t - 2 * W, t + 3):
        r2 = ring.copy()
        r2[p % wc] += 10
        out = pipeline.attend_row(q, kv, [1, 3], r2, wc, W, t, sink, 0.5)
        inside = any((pp % wc) == (p % wc) for pp in range(t - W + 1, t + 1))
        assert (np.abs(out - base).max() > 1e-6) == inside


def test_window_clamps_at_zero_and_k0_is_sliding_window():
    q, ring, sink = rnd(2, 4, seed=17), rnd(8, 4, seed=18), rnd(2, seed=19)
    rows = csa.attention_rows(np.zeros((0, 4)), [], ring, 8, 6, 2)
    np.testing.assert_array_equal(rows, ring[:3])          # positions 0..2 only
    o = pipeline.attend_row(q, np.zeros((0, 4)), [], ring, 8, 6, 2, sink, 0.5)
    np.testing.assert_allclose(o, sdpa(q, ring[:3], 0.5, sink), rtol=1e-12)
    # K = 0 and W = 0: no row at all -> 0
    assert np.all(pipeline.attend_row(q, np.zeros((0, 4)), [], ring, 8, 0, 5, sink, 0.5) == 0)


def test_selected_and_window_rows_are_both_kept():
    # the same vector as a selected entry and as a window row counts twice
    v = rnd(1, 4, seed=20)
    q = rnd(1, 4, seed=21)
    ring = np.repeat(v, 4, 0)
    o = pipeline.attend_row(q, v, [0], ring, 4, 1, 3, np.array([0.0]), 1.0)
    z = q[0] @ v[0]
    np.testing.assert_allclose(o[0], v[0] * 2 * np.exp(z) / (2 * np.exp(z) + 1), rtol=1e-13)


def test_sparse_equals_dense_when_all_visible_selected():
    # K >= n_vis with every visible entry selected == dense attention over all of them
    rng = np.random.default_rng(22)
    kv, k_idx = rng.standard_normal((50, 16)), rng.standard_normal((50, 8))
    q_idx, w = rng.standard_normal((3, 8)), rng.standard_normal(3)
    q, sink, ring = rng.standard_normal((4, 16)), rng.standard_normal(4), rng.standard_normal((32, 16))
    t, m = 101, 4
    n = csa.n_visible(t, m)
    ids, _, _ = pipeline.index_topk_row(q_idx, w, k_idx, t, m, 50, 64)
    assert ids[ids >= 0].tolist() == list(range(n))
    o = pipeline.attend_row(q, kv, ids, ring, 32, 8, t, sink, 0.25)
    dense = np.vstack([kv[:n], ring[[(p % 32) for p in range(t - 7, t + 1)]]])
    np.testing.assert_allclose(o, sdpa(q, dense, 0.25, sink), rtol=1e-11)
