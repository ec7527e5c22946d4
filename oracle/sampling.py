"""Column samples for ApproxD and row-norm samples of V (test infrastructure only).

HA page:

* section "Method overview": the product of the softmax matrix with V is
  approximated by a sampling matrix S built from the row norms of V; D can be
  estimated with uniform sampling instead of KDE-based importance sampling.
* section "Algorithm": D^-1 A times V is approximated by sampling according to
  the squared row l2 norms of V; ApproxD (Algorithm 2) combines the masked
  entries with a randomly chosen subset of columns of A.

Readings taken (the equations and listings were lost):

* Two independent draws of m samples each, one per purpose, both with
  replacement and shared by every query row of a sub-problem.
* Uniform columns: l_t = lo + floor(u_t n_k / 2^32), u_t the top 32 bits of
  draw(UNIFORM, head, node, t); every sample weighs alpha = n_k / m.
* V-row-norm samples: a_j = fp64 sum of v_jt^2 in order t = 0..d-1 (exact
  squares), M = max_j a_j over the head, integer weights
  W_j = ceil(2^32 a_j / M) (0 iff V_j = 0), P the exclusive prefix sum of W
  over the head, T = P[hi] - P[lo] for key range [lo, hi). Draw
  U_t = floor(R_t T / 2^64) with R_t = draw(VNORM, head, node, t) and take the
  least j with P[j+1] - P[lo] > U_t, i.e. p_j = W_j / T. The sample weighs
  T / (m W_j) (fp64: T / (m * W_j) with m and W_j converted, then rounded to
  fp32), which makes the sampled product unbiased.
* When m >= n_k the "sample" is every key of the range once with weight 1.
  When T = 0 (all V rows of the range are zero) the V list is empty.
"""

import numpy as np

from . import rng


def uniform_samples(seed, head, node, lo, n_k, m):
    """(indices [global], weight alpha) of the uniform column sample."""
    if m >= n_k:
        return np.arange(lo, lo + n_k, dtype=np.int64), 1.0
    idx = np.empty(m, dtype=np.int64)
    for t in range(m):
        u = rng.draw(seed, rng.PURPOSE_UNIFORM, head, node, t) >> 32
        idx[t] = lo + ((u * n_k) >> 32)
    return idx, n_k / m


def row_sq_norms(V):
    """a_j = v_j0^2 + v_j1^2 + ... summed left to right in fp64."""
    V = np.asarray(V, dtype=np.float64)
    a = np.zeros(V.shape[0])
    for t in range(V.shape[1]):
        a = a + V[:, t] * V[:, t]
    return a


def vnorm_weights(V):
    """Integer sampling weights W_j and their exclusive prefix sums P (uint64)."""
    a = row_sq_norms(V)
    M = a.max() if len(a) else 0.0
    W = np.zeros(len(a), dtype=np.uint64)
    if M > 0:
        # a / M is one rounded fp64 division; times 2^32 and ceil are exact
        W = np.ceil(2.0 ** 32 * (a / M)).astype(np.uint64)
    P = np.zeros(len(a) + 1, dtype=np.uint64)
    P[1:] = np.cumsum(W, dtype=np.uint64)
    return a, W, P


def vnorm_samples(seed, head, node, lo, n_k, P, W, m):
    """(indices [global], fp32 weights) of the V-row-norm sample."""
    if m >= n_k:
        return (np.arange(lo, lo + n_k, dtype=np.int64),
                np.ones(n_k, dtype=np.float32))
    base = int(P[lo])
    T = int(P[lo + n_k]) - base
    if T == 0:
        return np.zeros(0, dtype=np.int64), np.zeros(0, dtype=np.float32)
    rel = P[lo + 1: lo + n_k + 1].astype(np.uint64) - np.uint64(base)
    idx = np.empty(m, dtype=np.int64)
    w = np.empty(m, dtype=np.float32)
    for t in range(m):
        R = rng.draw(seed, rng.PURPOSE_VNORM, head, node, t)
        U = (R * T) >> 64
        # least local j with P[lo+j+1] - P[lo] > U
        j = int(np.searchsorted(rel, np.uint64(U), side="right"))
        idx[t] = lo + j
        w[t] = np.float32(float(T) / (float(m) * float(int(W[lo + j]))))
    return idx, w
