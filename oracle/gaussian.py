"""Standard normal values from two 64-bit draws (test infrastructure only).

The HA page's hash (section "Algorithm", Definition 1, read as signs of
projections on Gaussian hyperplanes) needs r Gaussian vectors per head, but
the page fixes no generator. The reading taken here makes the value of every
hyperplane entry a fixed number that any platform with IEEE-754 binary64
arithmetic reproduces bit for bit, so that a device can draw the hyperplanes
itself from the seed and still agree exactly with an independent host
implementation.

Box-Muller (Box and Muller, 1958): g = sqrt(-2 ln u1) cos(2 pi u2), with
u1 = ((a >> 11) + 1) 2^-53 in (0, 1] and u2 = (b >> 11) 2^-53 in [0, 1).
The three functions are evaluated with nothing but correctly rounded binary64
additions, subtractions, multiplications and divisions, in the fixed order
written below, on exactly split exponents (no fused multiply-add, no library
transcendental):

ln(u), u in (0, 1]   u = f 2^e with f in [1, 2); if f > SQRT2 then f = f/2,
                     e = e + 1. s = (f - 1) / (f + 1), z = s s,
                     p = Horner in z of the coefficients 1/(2k+1), k = 11..0
                     (the atanh series: ln f = 2 atanh s = 2 s sum z^k/(2k+1)),
                     ln u = e LN2 + (2 s) p.
sqrt(y), y > 0       y = m 2^e with m in [1, 2); if e is odd then m = 2 m,
                     e = e - 1. x = (1 + m) / 2, then six Newton steps
                     x = (x + m / x) / 2; sqrt y = x 2^(e/2). y = 0 gives 0.
cos(2 pi u)          with B = b >> 11 (u = B 2^-53): q = (B + 2^50) >> 51
                     (the quadrant nearest to 4u), r = (B - q 2^51) 2^-51 in
                     [-1/2, 1/2), theta = r PIO2, t = theta theta,
                     C = Horner in t of (-1)^k/(2k)!, k = 9..0 (cos theta),
                     S = theta * Horner in t of (-1)^k/(2k+1)!, k = 8..0
                     (sin theta); cos 2 pi u = C, -S, -C, S for q mod 4 =
                     0, 1, 2, 3.
g                    = sqrt(-2 ln u1) * cos 2 pi u2 (one product), then
                     rounded to fp32 and to the nearest bfloat16 (ties to
                     even) by the caller.

The constants are the binary64 values nearest to the decimals below (LN2,
SQRT2, PIO2, and the series coefficients). Truncating the series where
written keeps every function within a few binary64 ulps of the true value,
which tests/test_oracle_gaussian.py checks against the C library.

numpy's float64 arithmetic is elementwise IEEE-754 with round to nearest, so
this module follows the definition directly.
"""

import numpy as np

from . import rng

LN2 = 0.6931471805599453094          # ln 2
SQRT2 = 1.4142135623730950488        # sqrt 2
PIO2 = 1.5707963267948966192         # pi / 2
LN_COEF = [1.0 / (2 * k + 1) for k in range(12)]            # 1, 1/3, ..., 1/23
COS_COEF = [(-1.0) ** k / float(np.prod(np.arange(1, 2 * k + 1, dtype=np.float64)))
            for k in range(10)]                               # 1, -1/2!, ..., 1/18!
SIN_COEF = [(-1.0) ** k / float(np.prod(np.arange(1, 2 * k + 2, dtype=np.float64)))
            for k in range(9)]                                # 1, -1/3!, ..., 1/17!
NEWTON_STEPS = 6


def _split(x):
    """x = f 2^e exactly, with f in [1, 2) (x > 0 and normal)."""
    f, e = np.frexp(np.asarray(x, dtype=np.float64))    # f in [0.5, 1)
    return f * 2.0, e.astype(np.int64) - 1


def ln_unit(u):
    """ln u for u in (0, 1], as defined in the module docstring."""
    f, e = _split(u)
    big = f > SQRT2
    f = np.where(big, f * 0.5, f)
    e = np.where(big, e + 1, e)
    s = (f - 1.0) / (f + 1.0)
    z = s * s
    p = np.full_like(z, LN_COEF[11])
    for k in range(10, -1, -1):
        p = p * z + LN_COEF[k]
    return e.astype(np.float64) * LN2 + (2.0 * s) * p


def sqrt_newton(y):
    """sqrt y for y >= 0, as defined in the module docstring."""
    y = np.asarray(y, dtype=np.float64)
    pos = y > 0
    m, e = _split(np.where(pos, y, 1.0))
    odd = (e & 1) == 1
    m = np.where(odd, m * 2.0, m)
    e = np.where(odd, e - 1, e)
    x = (1.0 + m) / 2.0
    for _ in range(NEWTON_STEPS):
        x = (x + m / x) / 2.0
    return np.where(pos, np.ldexp(x, e // 2), 0.0)


def cos_two_pi(B):
    """cos(2 pi B 2^-53) for integers 0 <= B < 2^53 (uint64 array)."""
    B = np.asarray(B, dtype=np.uint64)
    q = (B + np.uint64(1 << 50)) >> np.uint64(51)
    r = (B.astype(np.int64) - (q.astype(np.int64) << 51)).astype(np.float64) * 2.0 ** -51
    theta = r * PIO2
    t = theta * theta
    C = np.full_like(t, COS_COEF[9])
    for k in range(8, -1, -1):
        C = C * t + COS_COEF[k]
    S = np.full_like(t, SIN_COEF[8])
    for k in range(7, -1, -1):
        S = S * t + SIN_COEF[k]
    S = theta * S
    quad = (q & np.uint64(3)).astype(np.int64)
    return np.select([quad == 0, quad == 1, quad == 2], [C, -S, -C], S)


def box_muller(a, b):
    """g (fp64) from the 64-bit draws a, b (uint64 arrays)."""
    a = np.asarray(a, dtype=np.uint64)
    b = np.asarray(b, dtype=np.uint64)
    u1 = ((a >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * 2.0 ** -53
    R = sqrt_newton(-2.0 * ln_unit(u1))
    return R * cos_two_pi(b >> np.uint64(11))


def hyperplane_draws(seed, heads, r, d):
    """The two draws (a, b) of every hyperplane entry: entry (h, k, t) takes
    counters 2e and 2e + 1, e = k d + t, of purpose "hyperplane", node 0."""
    a = np.empty((heads, r, d), dtype=np.uint64)
    b = np.empty((heads, r, d), dtype=np.uint64)
    for h in range(heads):
        for k in range(r):
            for t in range(d):
                e = k * d + t
                a[h, k, t] = rng.draw(seed, rng.PURPOSE_HYPERPLANE, h, 0, 2 * e)
                b[h, k, t] = rng.draw(seed, rng.PURPOSE_HYPERPLANE, h, 0, 2 * e + 1)
    return a, b
