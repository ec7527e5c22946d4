"""Rows whose projection on one hyperplane sits at a chosen multiple of the
hash kernel's certainty margin (test inputs, not part of the oracle).

The kernel trusts the fp32 sign of <x, g_k> when its magnitude exceeds
3 gamma_d sum_t |x_t g_kt| (bf16 rows, projections on MFMA) or
4 gamma_d |x| |g_k| (fp32 rows), gamma_d = d u / (1 - d u), u = 2^-24, and
otherwise recomputes the fp64 sequential sum. Rows at 0.5, 1, 2 and 10 times
that margin exercise both sides of the decision."""

import numpy as np

from oracle import sortlsh as osl


def _seqdot(X, g):
    p = np.zeros(X.shape[0])
    for t in range(X.shape[1]):
        p = p + X[:, t] * g[t]
    return p


def margin(X, g, dtype):
    d = len(g)
    u = 2.0 ** -24
    gam = d * u / (1 - d * u)
    if dtype == "bf16":
        return 3 * gam * (np.abs(X) @ np.abs(g))
    return 4 * gam * np.linalg.norm(X, axis=1) * np.linalg.norm(g)


def rows_at_margin(G, k, c, sign, count, rs, dtype):
    """`count` random rows (bf16 or fp32 values, as fp64) with
    <x, g_k> = sign * (about c) * margin; returns (rows, ratios)."""
    d = G.shape[1]
    g = G[k].astype(np.float64)
    if dtype == "bf16":
        def rnd(x):
            return osl.round_bf16_array(np.asarray(x, dtype=np.float32)).astype(np.float64)
    else:
        def rnd(x):
            return np.asarray(x, dtype=np.float32).astype(np.float64)
    N = count * 40
    X = rnd(rs.standard_normal((N, d)))
    order = np.argsort(-np.abs(g))
    j, t2 = order[0], order[1]          # coarse and fine adjustment coordinates
    X[:, t2] = rnd(0.01 * rs.standard_normal(N))
    for _ in range(3):
        p = _seqdot(X, g)
        X[:, j] = rnd(X[:, j] - (p - sign * c * margin(X, g, dtype)) / g[j])
        p = _seqdot(X, g)
        X[:, t2] = rnd(X[:, t2] - (p - sign * c * margin(X, g, dtype)) / g[t2])
    ratio = _seqdot(X, g) / margin(X, g, dtype)
    ok = (np.sign(ratio) == sign) & (np.abs(ratio) > 0.8 * c) & (np.abs(ratio) < 1.25 * c)
    return X[ok][:count], ratio[ok][:count]


def margin_set(seed, d, dtype, per_cell=16, rs_seed=0):
    """Rows for every hyperplane of head 0, c in (0.5, 1, 2, 10), both signs."""
    G = osl.hyperplanes(seed, 1, 8, d)[0]
    rs = np.random.default_rng(rs_seed)
    rows, ratios = [], []
    for k in range(8):
        for c in (0.5, 1.0, 2.0, 10.0):
            for sign in (1, -1):
                X, r = rows_at_margin(G, k, c, sign, per_cell, rs, dtype)
                rows.append(X)
                ratios.append(np.stack([np.full(len(r), k), np.full(len(r), c), r], axis=1))
    return G, np.concatenate(rows), np.concatenate(ratios)
