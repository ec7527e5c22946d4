"""Pins of the oracle's Gaussian (oracle/gaussian.py) to mathematics it does
not share: each of ln, sqrt and cos against 50-digit mpmath values, the
Box-Muller values against the C library's formula, and the distribution
against N(0, 1)."""

import math

import mpmath
import numpy as np
import pytest

from oracle import gaussian, rng

mpmath.mp.dps = 50


def _ulps(got, exact):
    """|got - exact| in units of the last place of the exact value."""
    out = []
    for g, e in zip(got, exact):
        e = mpmath.mpf(e)
        ulp = math.ulp(float(abs(e))) if e != 0 else 2.0 ** -1074
        out.append(float(abs(mpmath.mpf(float(g)) - e)) / ulp)
    return np.array(out)


def _unit_points(count, seed):
    rs = np.random.default_rng(seed)
    B = rs.integers(0, 1 << 53, count, dtype=np.uint64)
    u = (B + np.uint64(1)).astype(np.float64) * 2.0 ** -53
    sq = math.sqrt(2.0) / 2.0
    edges = [1.0, 2.0 ** -53, 0.5, np.nextafter(sq, 0), sq, np.nextafter(sq, 1),
             np.nextafter(1.0, 0), 0.75, 0.25 + 2.0 ** -53]
    return np.concatenate([u, np.array(edges)])


def test_ln_within_four_ulps_of_the_exact_logarithm():
    u = _unit_points(3000, 1)
    got = gaussian.ln_unit(u)
    exact = [mpmath.log(mpmath.mpf(float(x))) for x in u]
    err = _ulps(got, exact)
    ok = np.array([float(x) != 1.0 for x in u])
    assert err[ok].max() <= 4.0, err.max()
    assert gaussian.ln_unit(np.array([1.0]))[0] == 0.0


def test_sqrt_within_one_ulp_of_the_exact_root():
    rs = np.random.default_rng(2)
    y = np.concatenate([rs.uniform(0, 80, 3000), rs.uniform(0, 1e-12, 200),
                        np.array([2.0 ** -52, 1.0, 2.0, 4.0, 0.5, 74.5, np.nextafter(4.0, 0)])])
    got = gaussian.sqrt_newton(y)
    exact = [mpmath.sqrt(mpmath.mpf(float(x))) for x in y]
    assert _ulps(got, exact).max() <= 1.0
    assert gaussian.sqrt_newton(np.array([0.0, -0.0]))[0] == 0.0
    # perfect squares come out exact
    sq = np.arange(1, 200, dtype=np.float64)
    assert np.array_equal(gaussian.sqrt_newton(sq * sq), sq)


def test_cos_two_pi_against_the_exact_angle():
    """cos(2 pi u) for u = B 2^-53 exactly: absolute error below 4e-16 (the
    argument is exact, so this also checks the quadrant logic)."""
    rs = np.random.default_rng(3)
    B = rs.integers(0, 1 << 53, 3000, dtype=np.uint64)
    quarter = 1 << 51
    edges = [0, 1, quarter - 1, quarter, quarter + 1, 2 * quarter, 3 * quarter,
             (quarter >> 1) - 1, quarter >> 1, 7 * (quarter >> 1), (1 << 53) - 1]
    B = np.concatenate([B, np.array(edges, dtype=np.uint64)])
    got = gaussian.cos_two_pi(B)
    for g, b in zip(got, B):
        exact = mpmath.cos(2 * mpmath.pi * mpmath.mpf(int(b)) / mpmath.mpf(2) ** 53)
        assert abs(mpmath.mpf(float(g)) - exact) < 4e-16, (int(b), float(g))
    assert gaussian.cos_two_pi(np.array([0], dtype=np.uint64))[0] == 1.0
    assert gaussian.cos_two_pi(np.array([2 * quarter], dtype=np.uint64))[0] == -1.0


def test_box_muller_matches_the_library_formula():
    """g agrees with sqrt(-2 log u1) cos(2 pi u2) of the C library to 1e-13
    relative to max(1, |g|) (the C library's cos sees 2 pi u2 rounded)."""
    rs = np.random.default_rng(4)
    a = rs.integers(0, 2 ** 64, 20000, dtype=np.uint64, endpoint=False)
    b = rs.integers(0, 2 ** 64, 20000, dtype=np.uint64, endpoint=False)
    g = gaussian.box_muller(a, b)
    u1 = ((a >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * 2.0 ** -53
    u2 = (b >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    ref = np.array([math.sqrt(-2.0 * math.log(x)) * math.cos(2.0 * math.pi * y)
                    for x, y in zip(u1, u2)])
    assert np.max(np.abs(g - ref) / np.maximum(1.0, np.abs(ref))) < 1e-13
    # u1 = 1 (a >> 11 all ones) gives radius 0
    top = np.array([2 ** 64 - 1], dtype=np.uint64)
    assert gaussian.box_muller(top, np.array([5], dtype=np.uint64))[0] == 0.0


def test_box_muller_is_standard_normal():
    from scipy import stats
    a = np.array([rng.draw(77, rng.PURPOSE_HYPERPLANE, 0, 0, 2 * e) for e in range(20000)],
                 dtype=np.uint64)
    b = np.array([rng.draw(77, rng.PURPOSE_HYPERPLANE, 0, 0, 2 * e + 1) for e in range(20000)],
                 dtype=np.uint64)
    g = gaussian.box_muller(a, b)
    assert abs(g.mean()) < 5 / math.sqrt(g.size)
    assert abs(g.var() - 1.0) < 5 * math.sqrt(2.0 / g.size)
    assert stats.kstest(g, "norm").pvalue > 1e-4


@pytest.mark.parametrize("planted", ["ln", "cos"])
def test_a_wrong_term_is_caught(planted, monkeypatch):
    """A dropped series term shows up in the pins above (checked here by
    planting one on the CPU)."""
    if planted == "ln":
        monkeypatch.setattr(gaussian, "LN_COEF", gaussian.LN_COEF[:-3] + [0.0, 0.0, 0.0])
        u = _unit_points(500, 5)
        err = _ulps(gaussian.ln_unit(u), [mpmath.log(mpmath.mpf(float(x))) for x in u])
        assert err.max() > 4.0
    else:
        monkeypatch.setattr(gaussian, "COS_COEF", gaussian.COS_COEF[:-2] + [0.0, 0.0])
        B = np.array([(1 << 50) - 1], dtype=np.uint64)   # theta just under pi/4 (quadrant 0)
        exact = mpmath.cos(mpmath.pi / 4)
        assert abs(mpmath.mpf(float(gaussian.cos_two_pi(B)[0])) - exact) > 4e-16
