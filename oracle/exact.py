"""Exact softmax attention in fp64 (test infrastructure only).

HA page, section "Method overview": Q, K, V are n x d; A := exp(QK^T)
elementwise; D is the n x n diagonal matrix of the row sums of A; D^-1 A is
the softmax matrix and the output is Att = D^-1 A V. Computing it directly
costs Theta(n^2 d) time.

Reading taken (the page's formula for the output was lost in extraction):
Att = D^-1 A V, with the scores scaled by 1/sqrt(d) (the usual attention
scale; the workloads state it), i.e. A_ij = exp(<q_i, k_j> / sqrt(d)).

The causal mask M^C (section "Algorithm", Figure 2) keeps key j for query i
iff j <= i.

Besides O the functions return lse_i = log(D_ii) (natural log, scaled
scores), the row's log-normaliser. Subtracting the row maximum before exp is
the usual overflow guard; it cancels exactly in D^-1 A.
"""

import numpy as np


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def exact_attention(Q, K, V, causal=False, scale=None):
    """Att = D^-1 exp(Q K^T * scale) V for one head. Q, K, V: [n, d]."""
    Q, K, V = _as64(Q), _as64(K), _as64(V)
    n, d = Q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    S = (Q @ K.T) * scale
    if causal:
        i = np.arange(n)[:, None]
        j = np.arange(K.shape[0])[None, :]
        S = np.where(j <= i, S, -np.inf)
    c = S.max(axis=1, keepdims=True)
    A = np.exp(S - c)                 # A scaled by exp(-c_i) per row
    Dii = A.sum(axis=1, keepdims=True)
    O = (A @ V) / Dii
    lse = c[:, 0] + np.log(Dii[:, 0])
    return O, lse


def exact_attention_rows(Q, K, V, rows, causal=False, scale=None):
    """Exact attention for the listed query rows only (same definition)."""
    Q, K, V = _as64(Q), _as64(K), _as64(V)
    rows = np.asarray(rows, dtype=np.int64)
    d = Q.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    O = np.empty((len(rows), V.shape[1]))
    lse = np.empty(len(rows))
    for t, i in enumerate(rows):
        hi = i + 1 if causal else K.shape[0]
        s = (K[:hi] @ Q[i]) * scale
        c = s.max()
        a = np.exp(s - c)
        O[t] = (a @ V[:hi]) / a.sum()
        lse[t] = c + np.log(a.sum())
    return O, lse


def lse_merge(parts):
    """Combine normalised partial results over disjoint key sets.

    Each part is (O_p, lse_p) with O_p = sum_j a_j v_j / sum_j a_j over its key
    set and lse_p = log sum_j a_j. Over the union, with L = log sum_p exp(lse_p),
    the output is sum_p exp(lse_p - L) O_p: the plain algebra of combining row
    sums, used for "merging attention outputs" (HA page, section "Single
    self-attention layer").
    """
    lses = np.stack([p[1] for p in parts])            # [P, rows]
    L = lses.max(axis=0) + np.log(np.exp(lses - lses.max(axis=0)).sum(axis=0))
    O = sum(np.exp(p[1] - L)[:, None] * p[0] for p in parts)
    return O, L
