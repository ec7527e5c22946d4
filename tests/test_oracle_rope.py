"""Pins of the oracle's rotary embedding (oracle/rope.py): closed forms and
invariants that a dropped term, a swapped sign or a wrong pairing would
break."""

import math

import numpy as np

from oracle import rope


def test_position_zero_is_identity():
    rs = np.random.default_rng(1)
    X = rope.round_bf16_array(rs.standard_normal((1, 64)).astype(np.float32))
    assert np.array_equal(rope.rope(X, dtype="bf16"), X)


def test_two_dimensional_rotation_closed_form():
    # d = 2: theta_0 = 1, so row i turns by i radians counter-clockwise
    X = np.tile(np.array([[1.0, 0.0]], dtype=np.float32), (4, 1))
    Y = rope.rope(X, dtype="fp32")
    for i in range(4):
        assert abs(Y[i, 0] - math.cos(i)) < 1e-7 and abs(Y[i, 1] - math.sin(i)) < 1e-7


def test_pairing_frequencies_and_norms():
    n, d = 9, 16
    c, s = rope.angle_table(n, d, 10000.0)
    half = d // 2
    for t in range(half):
        th = 10000.0 ** (-2.0 * t / d)
        assert abs(math.acos(max(-1.0, min(1.0, c[1, t]))) - th) < 1e-12
    # a unit vector on coordinate t moves only within the pair (t, t + d/2)
    X = np.zeros((n, d), dtype=np.float32)
    X[:, 3] = 1.0
    Y = rope.rope(X, dtype="fp32", table=(c, s))
    assert np.all(Y[:, [k for k in range(d) if k not in (3, 3 + half)]] == 0)
    assert np.allclose(Y[:, 3] ** 2 + Y[:, 3 + half] ** 2, 1.0, atol=1e-6)
    assert np.allclose(Y[:, 3 + half], s[:, 3], atol=1e-7)


def test_scores_depend_only_on_relative_position():
    rs = np.random.default_rng(2)
    d = 32
    q = rs.standard_normal(d).astype(np.float32)
    k = rs.standard_normal(d).astype(np.float32)
    n = 12
    Q = rope.rope(np.tile(q, (n, 1)), dtype="fp32").astype(np.float64)
    K = rope.rope(np.tile(k, (n, 1)), dtype="fp32").astype(np.float64)
    for delta in (0, 3, 7):
        vals = [Q[i + delta] @ K[i] for i in range(n - delta)]
        assert max(vals) - min(vals) < 1e-4 * (abs(vals[0]) + 1)


def test_bf16_rounding_of_the_fp32_result():
    vals = np.array([1.0, 1.00390625, 1.005859375, -2.5078125], dtype=np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 (ties to even -> 1);
    # 1 + 3 * 2^-9 rounds up to 1 + 2^-7
    assert np.array_equal(rope.round_bf16_array(vals),
                          np.array([1.0, 1.0, 1.0078125, -2.5], dtype=np.float32))
