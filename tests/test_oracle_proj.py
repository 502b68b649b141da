"""Pins for the oracle's grouped output projection: one group is the plain
product of the flattened head outputs with one matrix; G groups equal the
product with the block-diagonal matrix of the group weights (which fixes the
head-to-group assignment and the concatenation order); a hand-worked example."""
import numpy as np

from oracle import proj


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_one_group_is_the_plain_product():
    T, H, d, dg = 7, 4, 8, 5
    o, w = _rand((T, H, d), 0), _rand((1, dg, H * d), 1)
    np.testing.assert_allclose(proj.grouped_out_proj(o, w), o.reshape(T, H * d) @ w[0].T,
                               rtol=1e-13, atol=1e-13)


def test_groups_equal_block_diagonal_product():
    T, H, d, G, dg = 5, 6, 4, 3, 7
    o, w = _rand((T, H, d), 2), _rand((G, dg, (H // G) * d), 3)
    K = (H // G) * d
    bd = np.zeros((H * d, G * dg))
    for j in range(G):
        bd[j * K:(j + 1) * K, j * dg:(j + 1) * dg] = w[j].T
    np.testing.assert_allclose(proj.grouped_out_proj(o, w), o.reshape(T, H * d) @ bd,
                               rtol=1e-13, atol=1e-13)


def test_hand_worked_example():
    # T=1, H=2 heads of d=1, G=2 groups of one head, dg=2:
    # o = [3, -2];  W_0 = [[1], [2]],  W_1 = [[5], [-1]]  (rows = outputs)
    # y = [3*1, 3*2, -2*5, -2*-1] = [3, 6, -10, 2]
    o = np.array([[[3.0], [-2.0]]])
    w = np.array([[[1.0], [2.0]], [[5.0], [-1.0]]])
    np.testing.assert_array_equal(proj.grouped_out_proj(o, w), [[3.0, 6.0, -10.0, 2.0]])
