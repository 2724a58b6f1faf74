"""Pins for the output-projection oracle (CPU): y = o W^T + b.

Checked against the bias alone (o = 0), one-hot rows of o (exactly a row of
W plus the bias), linearity in o, and brute force with math.fsum (Perplexity,
"GPT-OSS on day 0", section "GPT-OSS on Hopper": the output projection has a
bias).
"""

import math

import numpy as np

from oracle import oproj_ref


def test_zero_input_gives_the_bias_and_one_hot_rows_pick_weight_columns():
    rng = np.random.default_rng(0)
    w = rng.standard_normal((6, 10))
    b = rng.standard_normal(6)
    assert np.array_equal(oproj_ref(np.zeros((3, 10)), w, b), np.tile(b, (3, 1)))
    eye = np.eye(10)
    assert np.array_equal(oproj_ref(eye, w, b), w.T + b[None, :])
    assert np.array_equal(oproj_ref(eye, w, None), w.T)


def test_linearity_and_brute_force():
    rng = np.random.default_rng(1)
    o1, o2 = rng.standard_normal((4, 12)), rng.standard_normal((4, 12))
    w = rng.standard_normal((5, 12))
    b = rng.standard_normal(5)
    lhs = oproj_ref(2.0 * o1 - o2, w, None)
    assert np.allclose(lhs, 2.0 * oproj_ref(o1, w, None) - oproj_ref(o2, w, None), rtol=0, atol=1e-12)
    y = oproj_ref(o1, w, b)
    for n in range(4):
        for e in range(5):
            assert abs(y[n, e] - (math.fsum(o1[n, k] * w[e, k] for k in range(12)) + b[e])) < 1e-12
