"""Pins for the oracle's backward pass (CPU only).

The gradients are pinned to central finite differences of the forward
oracle: every coordinate for a tiny exact case, and random directions for
HyperAttention with its buckets and samples held fixed. Two further pins are
the reductions to exact attention's gradient when the buckets cover the keys
or the recursion base covers n, and the shift invariance of the keys
(sum_j dK_j = 0).
"""

import numpy as np
import pytest

from oracle import backward as bw, exact, hyperattention as ha


def _fd(f, X, U, eps=1e-6):
    return (f(X + eps * U) - f(X - eps * U)) / (2 * eps)


@pytest.mark.parametrize("causal", [False, True])
def test_exact_gradient_every_coordinate(causal):
    rs = np.random.default_rng(11)
    n, d = 5, 3
    Q, K, V, dO = (rs.standard_normal((n, d)) for _ in range(4))
    grads = bw.exact_attention_backward(Q, K, V, dO, causal=causal)
    for which, G in enumerate(grads):
        for i in range(n):
            for t in range(d):
                U = np.zeros((n, d))
                U[i, t] = 1.0

                def loss(Xp):
                    X = [Q, K, V]
                    X[which] = Xp
                    return (exact.exact_attention(*X, causal=causal)[0] * dO).sum()

                fd = _fd(loss, [Q, K, V][which], U)
                assert abs(fd - G[i, t]) < 1e-8 * max(1.0, abs(fd)), (which, i, t)


def test_exact_gradient_identities():
    rs = np.random.default_rng(12)
    n, d = 40, 8
    Q, K, V, dO = (rs.standard_normal((n, d)) for _ in range(4))
    for causal in (False, True):
        dQ, dK, dV = bw.exact_attention_backward(Q, K, V, dO, causal=causal)
        # adding one vector to every key leaves each softmax row unchanged
        assert np.abs(dK.sum(axis=0)).max() < 1e-12 * np.abs(dK).max() * n
        # the rows of P sum to one, so the columns of dV sum to those of dO
        assert np.abs(dV.sum(axis=0) - dO.sum(axis=0)).max() < 1e-12 * n
    # constant V: the output does not depend on Q or K
    Vc = np.tile(rs.standard_normal(d), (n, 1))
    dQ, dK, _ = bw.exact_attention_backward(Q, K, Vc, dO, causal=True)
    assert np.abs(dQ).max() < 1e-12 and np.abs(dK).max() < 1e-12


CASES = [
    # non-causal, 4 buckets, both samples smaller than n (weights != 1)
    (True, dict(causal=False, b=16, m=8, r=4, seed=3)),
    # causal: 2 levels over n = 64, buckets of 8, base case 16
    (True, dict(causal=True, b=8, m=8, r=4, seed=5, recursion_base=16)),
    # causal with b covering the first level's half (one bucket, every sample
    # masked) and m covering the second's (every key once, weight 1)
    (False, dict(causal=True, b=32, m=16, r=3, seed=9, recursion_base=16)),
]


@pytest.mark.parametrize("mixed,kw", CASES)
def test_hyperattention_gradient_matches_finite_differences(mixed, kw):
    rs = np.random.default_rng(kw["seed"])
    H, n, d = 2, 64, 8
    Q, K, V, dO = (rs.standard_normal((H, n, d)) for _ in range(4))
    art = {}
    ha.hyperattention(Q, K, V, artifacts=art, **kw)
    if mixed:
        # masked and unmasked samples and non-unit V-norm weights
        bkts = np.concatenate([np.concatenate([s["u_bucket"], s["v_bucket"]])
                               for s in art["sub"][0]])
        assert len(np.unique(bkts)) > 1
        assert any(np.any(np.asarray(s["v_w"]) != 1.0) for s in art["sub"][0])
    grads = bw.hyperattention_backward(Q, K, V, dO, **kw)
    for which, G in enumerate(grads):
        for _ in range(2):
            U = rs.standard_normal((H, n, d))

            def loss(Xp):
                X = [Q, K, V]
                X[which] = Xp
                O, _ = ha.hyperattention(*X, sample_from=(Q, K, V), **kw)
                return (O * dO).sum()

            fd = _fd(loss, [Q, K, V][which], U)
            assert abs(fd - (G * U).sum()) < 1e-7 * max(1.0, abs(fd)), which
    # shift invariance of the keys holds for the estimator too
    dK = grads[1]
    assert np.abs(dK.sum(axis=1)).max() < 1e-12 * n * np.abs(dK).max()


def test_sample_from_inputs_is_the_default():
    rs = np.random.default_rng(4)
    Q, K, V = (rs.standard_normal((1, 64, 8)) for _ in range(3))
    kw = dict(causal=True, b=8, m=8, r=4, seed=1, recursion_base=16)
    O1, L1 = ha.hyperattention(Q, K, V, **kw)
    O2, L2 = ha.hyperattention(Q, K, V, sample_from=(Q, K, V), **kw)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_reduces_to_exact_gradient():
    rs = np.random.default_rng(8)
    H, n, d = 2, 64, 8
    Q, K, V, dO = (rs.standard_normal((H, n, d)) for _ in range(4))
    # one bucket holds every key: every sample lies in the query's bucket
    g = bw.hyperattention_backward(Q, K, V, dO, causal=False, b=n, m=8, r=4, seed=2)
    # recursion base covering n: the base case is the whole causal problem
    gc = bw.hyperattention_backward(Q, K, V, dO, causal=True, b=8, m=8, r=4, seed=2,
                                    recursion_base=n)
    for h in range(H):
        e = bw.exact_attention_backward(Q[h], K[h], V[h], dO[h], causal=False)
        ec = bw.exact_attention_backward(Q[h], K[h], V[h], dO[h], causal=True)
        for a, x in zip(g, e):
            assert np.abs(a[h] - x).max() < 1e-12
        for a, x in zip(gc, ec):
            assert np.abs(a[h] - x).max() < 1e-12


@pytest.mark.parametrize("kw", [c[1] for c in CASES])
def test_row_gradients_equal_full_gradients(kw):
    """The row-restricted gradients (used at full problem sizes) equal the
    full backward pass's rows, including keys drawn as samples."""
    rs = np.random.default_rng(21)
    H, n, d = 2, 64, 8
    Q, K, V, dO = (rs.standard_normal((H, n, d)) for _ in range(4))
    art = {}
    ha.hyperattention(Q, K, V, artifacts=art, **kw)
    sampled = np.unique(np.concatenate([np.concatenate([s["u_idx"], s["v_idx"]])
                                        for s in art["sub"][0]]))
    q_rows = np.array([0, 5, 31, 32, 47, 63])
    k_rows = np.unique(np.concatenate([[0, 17, 40, 63], sampled[:4]]))
    gq, gk, gv = bw.hyperattention_backward_rows(Q, K, V, dO, q_rows, k_rows, **kw)
    fq, fk, fv = bw.hyperattention_backward(Q, K, V, dO, **kw)
    assert np.abs(gq - fq[:, q_rows]).max() < 1e-12 * max(1.0, np.abs(fq).max())
    assert np.abs(gk - fk[:, k_rows]).max() < 1e-12 * max(1.0, np.abs(fk).max())
    assert np.abs(gv - fv[:, k_rows]).max() < 1e-12 * max(1.0, np.abs(fv).max())
