"""Pins for the oracle's indexer score and top-k: pure-Python brute force,
exact power-of-two rescaling, planted ties and the k >= n_e special case."""
import numpy as np
import pytest

from oracle import csa


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_scores_brute_force_loops():
    Tq, HI, dI, N = 3, 2, 5, 7
    qi, kic = _rand((Tq, HI, dI), 0), _rand((N, dI), 1)
    w = np.abs(_rand((Tq, HI), 2))
    s = csa.indexer_scores(qi, w, kic)
    for t in range(Tq):
        for j in range(N):
            tot = 0.0
            for h in range(HI):
                dot = 0.0
                for c in range(dI):
                    dot += qi[t, h, c] * kic[j, c]
                tot += w[t, h] * (dot if dot > 0 else 0.0)
            assert abs(s[t, j] - tot) < 1e-12


def test_single_head_unit_weight_is_relu_dot():
    qi, kic = _rand((4, 1, 8), 3), _rand((11, 8), 4)
    s = csa.indexer_scores(qi, np.ones((4, 1)), kic)
    ref = np.array([[max(0.0, float(np.dot(qi[t, 0], kic[j]))) for j in range(11)]
                    for t in range(4)])
    np.testing.assert_allclose(s, ref, rtol=1e-14, atol=0)
    assert np.all(s >= 0)


def test_power_of_two_weight_scaling_is_exact():
    qi, kic = _rand((2, 4, 16), 5), _rand((300, 16), 6)
    w = np.abs(_rand((2, 4), 7))
    s1 = csa.indexer_scores(qi, w, kic)
    s2 = csa.indexer_scores(qi, 2.0 * w, kic)
    assert np.array_equal(2.0 * s1, s2)
    for t in range(2):
        assert np.array_equal(csa.topk(s1[t], 300, 17), csa.topk(s2[t], 300, 17))


@pytest.mark.parametrize("n_e,k", [(0, 4), (3, 8), (50, 8), (50, 50), (257, 32)])
def test_topk_against_python_sorted(n_e, k):
    s = np.round(np.abs(_rand(max(n_e, 1) + 5, n_e)), 1)   # coarse rounding plants ties
    got = csa.topk(s, n_e, k)
    ranked = sorted(range(n_e), key=lambda j: (-s[j], j))[: min(k, n_e)]
    want = sorted(ranked) + [-1] * (k - min(k, n_e))
    assert got.tolist() == want
    assert got.dtype == np.int32


def test_topk_all_equal_takes_lowest_indices():
    s = np.zeros(100)
    assert csa.topk(s, 100, 10).tolist() == list(range(10))


def test_topk_k_ge_ne_takes_every_eligible_entry():
    s = np.abs(_rand(64, 8))
    got = csa.topk(s, 40, 64)
    assert got[:40].tolist() == list(range(40)) and np.all(got[40:] == -1)


def test_topk_ignores_ineligible_entries():
    s = np.arange(20, dtype=float)        # the largest scores sit past n_e
    assert csa.topk(s, 10, 3).tolist() == [7, 8, 9]


def test_kth_score():
    s = np.array([0.5, 2.0, 1.0, 2.0])
    assert csa.kth_score(s, 4, 2) == 2.0
    assert csa.kth_score(s, 4, 3) == 1.0
    assert csa.kth_score(s, 4, 10) == 0.5
