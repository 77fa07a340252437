"""Pins of the oracle's index score, causal visibility, Top-K and hierarchical pool."""
import itertools

import numpy as np
import pytest

from oracle import csa
from golden_util import arr, load


def rnd(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- index score
def test_index_hand_worked():
    g = load("hand_worked.json")["index_scores"]
    s = csa.index_scores(arr(g["q_idx"]), arr(g["w"]), arr(g["k_idx"]))
    np.testing.assert_allclose(s, arr(g["expected"]), rtol=0, atol=1e-15)


def test_single_head_unit_gate_is_relu_dot():
    q, k = rnd(1, 16, seed=1), rnd(50, 16, seed=2)
    s = csa.index_scores(q, np.ones(1), k)
    brute = [max(0.0, sum(q[0, c] * k[j, c] for c in range(16))) for j in range(50)]
    np.testing.assert_allclose(s, brute, rtol=1e-13, atol=1e-15)


def test_basis_keys_read_single_channels():
    # K_s = e_s: score = sum_h w_h max(0, q[h, s]) (no dot product left)
    H, d = 5, 7
    q, w = rnd(H, d, seed=3), rnd(H, seed=4)
    s = csa.index_scores(q, w, np.eye(d))
    expect = [sum(w[h] * max(0.0, q[h, c]) for h in range(H)) for c in range(d)]
    np.testing.assert_allclose(s, expect, rtol=1e-14, atol=1e-15)


def test_linear_in_gate_and_homogeneous_in_key():
    q, k = rnd(8, 32, seed=5), rnd(40, 32, seed=6)
    w1, w2 = rnd(8, seed=7), rnd(8, seed=8)
    np.testing.assert_allclose(csa.index_scores(q, 2 * w1 - 3 * w2, k),
                               2 * csa.index_scores(q, w1, k) - 3 * csa.index_scores(q, w2, k),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(csa.index_scores(q, w1, 2.5 * k), 2.5 * csa.index_scores(q, w1, k),
                               rtol=1e-13, atol=1e-14)


def test_relu_vetoes_negative_heads():
    # a head whose dot product is negative contributes nothing, whatever its gate
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    k = np.array([[2.0, -3.0]])
    for w1 in (-5.0, 0.0, 7.0):
        assert csa.index_scores(q, np.array([0.5, w1]), k)[0] == pytest.approx(1.0)
    # negating the key flips which head is active (no symmetry under k -> -k)
    assert csa.index_scores(q, np.array([0.5, 2.0]), -k)[0] == pytest.approx(6.0)


def test_score_scale_bounds_score():
    q, k, w = rnd(8, 16, seed=9), rnd(30, 16, seed=10), rnd(8, seed=11)
    assert np.all(np.abs(csa.index_scores(q, w, k)) <= csa.score_scale(q, w, k) + 1e-15)


# ---------------------------------------------------------------- visibility
@pytest.mark.parametrize("t,m,e,expected", [
    (-1, 4, None, 0), (0, 4, None, 0), (2, 4, None, 0), (3, 4, None, 1), (4, 4, None, 1),
    (7, 4, None, 2), (127, 128, None, 1), (126, 128, None, 0), (5, 1, None, 6),
    (1048575, 4, None, 262144), (1048575, 4, 1000, 1000), (65535, 4, 16384, 16384),
])
def test_n_visible_table(t, m, e, expected):
    assert csa.n_visible(t, m, e) == expected


def test_n_visible_matches_entry_definition_by_brute_force():
    # entry i covers [m i, m(i+1)); visible iff its last position m(i+1)-1 <= t
    for m in (1, 2, 4, 8):
        for t in range(0, 40):
            brute = sum(1 for i in range(64) if m * (i + 1) - 1 <= t)
            assert csa.n_visible(t, m) == brute


def test_prefill_chunk_visible_pairs_closed_form():
    # sum_{t=a}^{b} floor((t+1)/4) by the closed form of a floor sum
    a, b, m = 126976, 131071, 4
    def F(n):  # sum_{u=1}^{n} floor(u/m)
        q, r = divmod(n, m)
        return m * q * (q - 1) // 2 + q * (r + 1)
    total = F(b + 1) - F(a)
    assert total == sum(csa.n_visible(t, m) for t in range(a, b + 1))
    assert total == 132_119_552


# ---------------------------------------------------------------- Top-K
def test_topk_hand_worked():
    for c in load("hand_worked.json")["topk"]["cases"]:
        got = csa.select_topk(arr(c["scores"]), c["K"])
        assert got.tolist() == c["expected"], c["why"]


def beats(si, i, sj, j):
    return si > sj or (si == sj and i < j)


@pytest.mark.parametrize("seed", range(30))
def test_topk_is_the_dominating_set(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 40))
    K = int(rng.integers(1, 12))
    s = rng.integers(-3, 4, size=n).astype(np.float64)    # many exact ties
    s[rng.random(n) < 0.2] = -0.0
    got = csa.select_topk(s, K)
    sel = [int(i) for i in got if i >= 0]
    assert got.shape == (K,)
    assert sel == sorted(sel) and len(set(sel)) == len(sel)
    assert len(sel) == min(K, n) and all(i == -1 for i in got[len(sel):])
    s32 = s.astype(np.float32).astype(np.float64)
    rest = set(range(n)) - set(sel)
    for i in sel:
        for j in rest:
            assert beats(s32[i], i, s32[j], j)


def test_topk_brute_force_enumeration():
    # among all K-subsets, the chosen one maximises the sorted (score, -index) sequence
    rng = np.random.default_rng(3)
    for _ in range(20):
        n, K = 7, 3
        s = rng.integers(0, 3, size=n).astype(np.float64)
        def key(sub):
            return sorted(((s[i], -i) for i in sub), reverse=True)
        best = max(itertools.combinations(range(n), K), key=key)
        assert csa.select_topk(s, K).tolist() == sorted(best)


def test_topk_with_global_ids():
    s = np.array([0.5, 2.0, 2.0, 1.0])
    ids = np.array([10, 40, 30, 99])
    # tie between ids 40 and 30 at 2.0 -> both in; K=2 keeps them; ties by id not position
    assert csa.select_topk(s, 2, index=ids).tolist() == [30, 40]
    assert csa.select_topk(s, 1, index=ids).tolist() == [30]


# ---------------------------------------------------------------- hierarchical pool
def test_pool_hand_worked():
    for c in load("hand_worked.json")["candidate_pool"]["cases"]:
        got = csa.candidate_pool(arr(c["scores"]), c["block_size"], c["max_blocks"])
        assert got.tolist() == c["expected"], c["why"]


@pytest.mark.parametrize("seed", range(20))
def test_pool_properties(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 200))
    bs = int(rng.integers(1, 9))
    mb = int(rng.integers(1, 12))
    s = rng.integers(-5, 6, size=n).astype(np.float64)
    pool = csa.candidate_pool(s, bs, mb)
    nb = (n + bs - 1) // bs
    blocks = sorted(set(int(p) // bs for p in pool))
    assert len(blocks) == min(mb, nb)
    # the pool is exactly the visible entries of the chosen blocks, ascending
    expect = [e for b in blocks for e in range(b * bs, min(n, (b + 1) * bs))]
    assert pool.tolist() == expect
    bmax = [max(s[b * bs:min(n, (b + 1) * bs)]) for b in range(nb)]
    for b in blocks:
        for c in set(range(nb)) - set(blocks):
            assert beats(bmax[b], b, bmax[c], c)


def test_pool_covering_everything_reduces_to_flat_selection():
    # when the block budget covers every block, stage 2 over the pool == flat Top-K
    rng = np.random.default_rng(5)
    q1, q2, w1, w2 = rng.standard_normal((4, 16)), rng.standard_normal((4, 16)), \
        rng.standard_normal(4), rng.standard_normal(4)
    k = rng.standard_normal((100, 16))
    pool = csa.candidate_pool(csa.index_scores(q1, w1, k), 8, 13)
    assert pool.tolist() == list(range(100))
    s2 = csa.index_scores(q2, w2, k[pool])
    assert csa.select_topk(s2, 20, index=pool).tolist() == \
        csa.select_topk(csa.index_scores(q2, w2, k), 20).tolist()


def test_block_maxima_partial_last_block():
    s = np.array([1.0, 2.0, 3.0, -4.0, -5.0])
    np.testing.assert_array_equal(csa.block_maxima(s, 2), [2.0, 3.0, -5.0])
