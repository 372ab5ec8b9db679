"""Pins of the oracle's pooling compressor (softmax over a block's positions plus a position bias).

Source of the method: yudonglee.me "DeepSeek-V4 详解" 2.2 Step 1 and 2.3 Step 1; deepseek.csdn.net
"一文搞懂 DeepSeek" section V4 改进一. The pages print no formula; these tests pin the reading by
closed forms, invariants and brute force.
"""
import math

import numpy as np

from oracle import csa_oracle as o


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_weights_sum_to_one_per_channel_and_lie_in_unit_interval():
    g = _rand((4, 7), 0) * 3
    w = o.pool_weights(g, _rand(4, 1))
    assert w.shape == (4, 7)
    np.testing.assert_allclose(w.sum(axis=0), 1.0, rtol=0, atol=1e-15)
    assert (w > 0).all() and (w < 1).all()


def test_closed_form_two_positions():
    # Logits (0, ln 3) give weights (1/4, 3/4); channel 1 swaps them, so a softmax over the wrong
    # axis or a per-channel bias would fail.
    g = np.array([[0.0, math.log(3.0)], [math.log(3.0), 0.0]])
    w = o.pool_weights(g, np.zeros(2))
    np.testing.assert_allclose(w, [[0.25, 0.75], [0.75, 0.25]], atol=1e-15)
    x = np.array([[4.0, 8.0], [8.0, 4.0]])
    e = o.compress(x, g, np.zeros(2), 2)
    np.testing.assert_allclose(e, [[7.0, 7.0]], atol=1e-14)


def test_m1_is_identity():
    x, g = _rand((9, 5), 2), _rand((9, 5), 3)
    np.testing.assert_array_equal(o.compress(x, g, np.array([0.7]), 1), x)


def test_constant_block_gives_constant():
    x = np.tile(np.array([[1.5, -2.0, 0.25]]), (8, 1))
    e = o.compress(x, _rand((8, 3), 4), _rand(4, 5), 4)
    np.testing.assert_allclose(e, x[:2], atol=1e-15)


def test_equal_logits_zero_bias_give_mean():
    x = _rand((12, 6), 6)
    g = np.full((12, 6), 0.37)
    e = o.compress(x, g, np.zeros(4), 4)
    np.testing.assert_allclose(e, x.reshape(3, 4, 6).mean(axis=1), atol=1e-15)


def test_large_bias_selects_position():
    x, g = _rand((8, 5), 7), _rand((8, 5), 8)
    for i in range(4):
        b = np.zeros(4)
        b[i] = 40.0
        e = o.compress(x, g, b, 4)
        np.testing.assert_allclose(e, x.reshape(2, 4, 5)[:, i], atol=1e-12)


def test_shift_invariance_of_logits():
    x, g = _rand((8, 5), 9), _rand((8, 5), 10)
    b = _rand(4, 11)
    shift = np.repeat(_rand((2, 5), 12), 4, axis=0)      # same shift for a block's rows
    np.testing.assert_allclose(o.compress(x, g + shift, b, 4), o.compress(x, g, b, 4), atol=1e-14)


def test_entry_within_block_range():
    x, g = _rand((40, 9), 13), _rand((40, 9), 14) * 4
    e = o.compress(x, g, _rand(4, 15), 4)
    blocks = x.reshape(10, 4, 9)
    assert (e >= blocks.min(axis=1) - 1e-15).all() and (e <= blocks.max(axis=1) + 1e-15).all()


def test_trailing_partial_block_dropped():
    x, g = _rand((10, 3), 16), _rand((10, 3), 17)
    e = o.compress(x, g, np.zeros(4), 4)
    assert e.shape == (2, 3)
    np.testing.assert_allclose(e, o.compress(x[:8], g[:8], np.zeros(4), 4), atol=0)


def test_brute_force_scalar_loops():
    m, n, d = 4, 5, 3
    x, g, b = _rand((m * n + 2, d), 18), _rand((m * n + 2, d), 19) * 2, _rand(m, 20)
    e = o.compress(x, g, b, m)
    for j in range(n):
        for c in range(d):
            a = [g[j * m + i, c] + b[i] for i in range(m)]
            z = sum(math.exp(t) for t in a)
            want = sum(math.exp(a[i]) / z * x[j * m + i, c] for i in range(m))
            assert abs(e[j, c] - want) < 1e-13


def test_e4m3_row_store():
    e_c = _rand((6, 32), 21) * 0.05
    e_c[3] = 0.0
    q, sigma = o.store_e4m3_rows(e_c)
    # The largest magnitude of each nonzero row maps exactly onto +-448.
    for r in (0, 1, 2, 4, 5):
        assert np.max(np.abs(q[r])) == 448.0
        # 448 sigma recovers the row's largest magnitude to fp32 rounding of the scale.
        amax = np.abs(e_c[r]).max()
        assert abs(448.0 * sigma[r] - amax) <= 2.0 ** -23 * amax
        # Relative error of a stored value is within half an e4m3 ulp (2^-4) plus the scale's.
        big = np.abs(e_c[r]) > 2.0 ** -6 * sigma[r]
        rel = np.abs(q[r] * sigma[r] - e_c[r])[big] / np.abs(e_c[r])[big]
        assert rel.max() <= 2.0 ** -4 + 1e-7
    assert sigma[3] == 0.0 and (q[3] == 0).all()


# ---- projection (fp32 workload): x = hidden . W_x, g = hidden . W_g -------------------------
# deepseek.csdn.net "一文搞懂 DeepSeek" section "V3 看家本领一：MLA": the cached latent is a
# down-projection of the token's input; the gate logits come from a second projection.

def test_project_hand_worked():
    # Worked by hand: row 0 of x = 1*[1,0] + 2*[0,1] + 0*[2,3] = [1, 2];
    # row 1 of x = 0*[1,0] + 1*[0,1] - 1*[2,3] = [-2, -2];
    # row 0 of g = 1*[0,1] + 2*[1,0] + 0*[1,1] = [2, 1]; row 1 of g = [1,0] - [1,1] = [0, -1].
    hidden = np.array([[1.0, 2.0, 0.0], [0.0, 1.0, -1.0]])
    w_x = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, 3.0]])
    w_g = np.array([[0.0, 1.0], [1.0, 0.0], [1.0, 1.0]])
    x, g = o.project(hidden, w_x, w_g)
    assert x.tolist() == [[1.0, 2.0], [-2.0, -2.0]]
    assert g.tolist() == [[2.0, 1.0], [0.0, -1.0]]


def test_project_permutation_weights():
    # W_x a 3-cycle permutation: column j of x is column pi(j) of hidden. A transposed weight
    # gives the inverse cycle, and swapping W_x and W_g gives the other matrix: both fail.
    hidden = _rand((5, 3), 30)
    pi = [2, 0, 1]
    w_x = np.zeros((3, 3))
    for j, s in enumerate(pi):
        w_x[s, j] = 1.0
    w_g = 2.0 * np.eye(3)
    x, g = o.project(hidden, w_x, w_g)
    np.testing.assert_array_equal(x, hidden[:, pi])
    np.testing.assert_array_equal(g, 2.0 * hidden)


def test_project_brute_force_loops():
    hidden, w_x, w_g = _rand((4, 6), 31), _rand((6, 3), 32), _rand((6, 3), 33)
    x, g = o.project(hidden, w_x, w_g)
    for t in range(4):
        for c in range(3):
            assert abs(x[t, c] - sum(hidden[t, i] * w_x[i, c] for i in range(6))) < 1e-13
            assert abs(g[t, c] - sum(hidden[t, i] * w_g[i, c] for i in range(6))) < 1e-13
