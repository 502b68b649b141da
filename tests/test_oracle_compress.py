"""Pins for oracle.csa.compress: closed forms of softmax-gated pooling and a
pure-Python brute force on tiny blocks; for compress_window: width m is block
compression, a zero gate gives the mean of the window's present rows, and a
dominant bias selects the row at that window position."""
import math

import numpy as np
import pytest

from oracle import csa


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_m1_is_identity():
    k, v, ki = _rand((9, 8), 0), _rand((9, 8), 1), _rand((9, 4), 2)
    kc, vc, kic = csa.compress(k, v, ki, _rand(8, 3), 1)
    assert np.array_equal(kc, k) and np.array_equal(vc, v) and np.array_equal(kic, ki)


def test_zero_gate_is_block_mean():
    k, v, ki = _rand((32, 8), 4), _rand((32, 8), 5), _rand((32, 4), 6)
    kc, vc, kic = csa.compress(k, v, ki, np.zeros(8), 4)
    np.testing.assert_allclose(kc, k.reshape(8, 4, 8).mean(axis=1), rtol=0, atol=1e-15)
    np.testing.assert_allclose(vc, v.reshape(8, 4, 8).mean(axis=1), rtol=0, atol=1e-15)
    np.testing.assert_allclose(kic, ki.reshape(8, 4, 4).mean(axis=1), rtol=0, atol=1e-15)


def test_dominant_positional_bias_picks_that_token():
    k, v = _rand((24, 8), 7), _rand((24, 8), 8)
    b = np.zeros(6)
    b[4] = 60.0
    kc, vc, _ = csa.compress(k, v, None, _rand(8, 9) * 0.1, 6, pos_bias=b)
    np.testing.assert_allclose(kc, k[4::6], atol=1e-20)
    np.testing.assert_allclose(vc, v[4::6], atol=1e-20)


def test_partial_block_dropped_and_T_equals_m():
    k, v = _rand((10, 8), 10), _rand((10, 8), 11)
    g = _rand(8, 12)
    a = csa.compress(k, v, None, g, 4)
    b = csa.compress(k[:8], v[:8], None, g, 4)
    assert a[0].shape == (2, 8)
    np.testing.assert_array_equal(a[0], b[0])
    one = csa.compress(k[:4], v[:4], None, g, 4)
    assert one[0].shape == (1, 8)


def test_convex_combination_bounds():
    k, v = _rand((64, 16), 13), _rand((64, 16), 14)
    kc, vc, _ = csa.compress(k, v, None, _rand(16, 15) * 3, 8)
    kb, vb = k.reshape(8, 8, 16), v.reshape(8, 8, 16)
    assert np.all(kc <= kb.max(axis=1) + 1e-15) and np.all(kc >= kb.min(axis=1) - 1e-15)
    assert np.all(vc <= vb.max(axis=1) + 1e-15) and np.all(vc >= vb.min(axis=1) - 1e-15)


def test_bias_shift_invariance():
    k, v = _rand((16, 8), 16), _rand((16, 8), 17)
    g = _rand(8, 18)
    b = _rand(4, 19)
    x = csa.compress(k, v, None, g, 4, pos_bias=b)
    y = csa.compress(k, v, None, g, 4, pos_bias=b + 3.0)
    np.testing.assert_allclose(x[0], y[0], rtol=1e-13)


@pytest.mark.parametrize("m", [2, 3, 5])
def test_brute_force_python_loops(m):
    T, d, dI = 4 * m + 1, 3, 2
    k, v, ki = _rand((T, d), 20 + m), _rand((T, d), 30 + m), _rand((T, dI), 40 + m)
    g, b = _rand(d, 50 + m), _rand(m, 60 + m)
    kc, vc, kic = csa.compress(k, v, ki, g, m, pos_bias=b)
    for j in range(T // m):
        logits = []
        for i in range(m):
            s = 0.0
            for c in range(d):
                s += float(k[j * m + i, c]) * float(g[c])
            logits.append(s + float(b[i]))
        z = sum(math.exp(x) for x in logits)
        wts = [math.exp(x) / z for x in logits]
        for c in range(d):
            assert abs(kc[j, c] - sum(wts[i] * k[j * m + i, c] for i in range(m))) < 1e-12
            assert abs(vc[j, c] - sum(wts[i] * v[j * m + i, c] for i in range(m))) < 1e-12
        for c in range(dI):
            assert abs(kic[j, c] - sum(wts[i] * ki[j * m + i, c] for i in range(m))) < 1e-12


def test_eligibility_counts_completed_blocks():
    assert csa.n_eligible(2, 4) == 0
    assert csa.n_eligible(3, 4) == 1
    assert csa.n_eligible(7, 4) == 2
    assert csa.n_eligible(131071, 4) == 32768


# ---- overlapping windows ----
def test_window_of_m_is_block_compression():
    rng = np.random.default_rng(40)
    T, d, dI, m = 37, 6, 4, 4
    k, v, ki = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, dI))
    g, b = rng.standard_normal(d), rng.standard_normal(m)
    got = csa.compress_window(k, v, ki, g, m, m, b)
    ref = csa.compress(k, v, ki, g, m, b)
    for x, y in zip(got, ref):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)


def test_window_without_gate_is_the_mean_of_present_rows():
    # zero gate and biases: every present row of the window has weight 1/count
    rng = np.random.default_rng(41)
    T, d, m, width = 20, 5, 4, 7
    k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    kc, vc, _ = csa.compress_window(k, v, None, np.zeros(d), m, width)
    np.testing.assert_allclose(kc[0], k[0:4].mean(axis=0), rtol=1e-13)    # rows -3..3: 0..3 present
    np.testing.assert_allclose(vc[1], v[1:8].mean(axis=0), rtol=1e-13)    # rows 1..7
    np.testing.assert_allclose(vc[4], v[13:20].mean(axis=0), rtol=1e-13)  # rows 13..19


def test_window_bias_indexes_window_positions():
    # a dominant bias on window position p selects row (j+1)m - width + p
    rng = np.random.default_rng(42)
    T, d, m, width = 24, 3, 4, 8
    k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    for p in (0, 3, 7):
        b = np.zeros(width)
        b[p] = 200.0
        kc, vc, _ = csa.compress_window(k, v, None, rng.standard_normal(d) * 0.1, m, width, b)
        for j in range(1, T // m):
            np.testing.assert_allclose(vc[j], v[(j + 1) * m - width + p], rtol=1e-9, atol=1e-12)
