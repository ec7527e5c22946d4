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


def test_adjoint_identity():
    """<R x, y> = <x, R^T y> for the rotation R of every row: a wrong sign,
    a swapped half or a forward turn in place of the backward one breaks it."""
    rs = np.random.default_rng(3)
    n, d = 40, 32
    X = rs.standard_normal((n, d))
    Y = rs.standard_normal((n, d))
    tab = rope.angle_table(n, d, 10000.0)
    # the forward rotation in fp64 straight from the table, pair by pair
    c, s = tab
    RX = np.empty_like(X)
    for t in range(d // 2):
        RX[:, t] = X[:, t] * c[:, t] - X[:, t + d // 2] * s[:, t]
        RX[:, t + d // 2] = X[:, t] * s[:, t] + X[:, t + d // 2] * c[:, t]
    lhs = np.einsum("ij,ij->i", RX, Y)
    rhs = np.einsum("ij,ij->i", X, rope.rope_adjoint(Y, table=tab))
    assert np.abs(lhs - rhs).max() < 1e-12 * np.abs(lhs).max()


def test_adjoint_inverts_the_rotation():
    """R^T R = I: the adjoint of the rotated rows gives the rows back (fp32
    rotation, fp64 adjoint: within a few fp32 steps)."""
    rs = np.random.default_rng(4)
    X = rs.standard_normal((64, 64)).astype(np.float32)
    Y = rope.rope(X, dtype="fp32")
    back = rope.rope_adjoint(Y.astype(np.float64))
    assert np.abs(back - X).max() < 1e-5
    # position 0 is the identity, also for the fp32 and bf16 forms
    Xb = rope.round_bf16_array(X[:1])
    assert np.array_equal(rope.rope_adjoint(Xb, dtype="bf16"), Xb)


def test_adjoint_two_dimensional_closed_form():
    # d = 2: row i = (cos i, sin i) turns back onto (1, 0)
    n = 5
    G = np.array([[math.cos(i), math.sin(i)] for i in range(n)])
    out = rope.rope_adjoint(G, base=10000.0)
    assert np.allclose(out, np.tile([1.0, 0.0], (n, 1)), atol=1e-15)


def test_adjoint_is_the_gradient_by_finite_differences():
    """d/dX of sum(G * rope(X)) is rope_adjoint(G), checked by central
    differences of the fp64 rotation on a few coordinates."""
    rs = np.random.default_rng(5)
    n, d = 6, 8
    tab = rope.angle_table(n, d, 10000.0)
    c, s = tab
    X = rs.standard_normal((n, d))
    G = rs.standard_normal((n, d))

    def f(Z):
        z1, z2 = Z[:, : d // 2], Z[:, d // 2:]
        return float(np.sum(G * np.concatenate([z1 * c - z2 * s, z1 * s + z2 * c], axis=1)))

    grad = rope.rope_adjoint(G, table=tab)
    h = 1e-6
    for i, j in ((0, 0), (3, 1), (5, 5), (2, 7)):
        E = np.zeros_like(X)
        E[i, j] = h
        fd = (f(X + E) - f(X - E)) / (2 * h)
        assert abs(fd - grad[i, j]) < 1e-7
