"""Gradients of exact attention and of the HyperAttention estimator
(test infrastructure only).

The HA page times the forward and backward passes together (section "Single
self-attention layer") but states no formula for the backward pass. Reading
taken: the backward pass is the exact gradient of the forward pass as
hyperattention.py computes it, with the hash codes, buckets, sample lists and
sample weights held fixed. All of these are piecewise constant in Q, K and V:
the codes are signs of projections, and the V-norm weights are integers
quantised from the row norms. So this is the true gradient almost everywhere.

Derivation. Every row i of the final output, after the causal merge, has the
form

    O_i = N_i / Z_i,   N_i = sum_j w_ij e^{s_ij} V_j,   Z_i = sum_j u_ij e^{s_ij}

over the key slots j that row i evaluates:

* a bucket key or a base-case key has w = u = 1;
* a uniform column sample outside the query's bucket has w = 0, u = alpha;
* a V-norm sample outside the query's bucket has w = its weight, u = 0;
* a sample inside the query's bucket has w = u = 0.

The merge of per-level partials only regroups these sums, and
ln Z_i = Lambda_i is the final lse. With the loss gradient dO_i and
Delta_i = dO_i . O_i, the chain rule gives, for each slot,

    ds_ij = e^{s_ij - Lambda_i} (w_ij dO_i . V_j - u_ij Delta_i)
    dV_j += w_ij e^{s_ij - Lambda_i} dO_i

and, since s_ij = scale <q_i, k_j>,

    dq_i += scale ds_ij k_j,   dk_j += scale ds_ij q_i.

A key drawn more than once contributes once per draw. For exact attention,
w = u = 1 on every unmasked key, so this is the usual softmax gradient with
P_ij = e^{s_ij - Lambda_i}.
"""

import numpy as np

from . import exact, hyperattention as ha


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def exact_attention_backward(Q, K, V, dO, causal=False, scale=None):
    """dQ, dK, dV of sum(dO * Att) for Att = D^-1 exp(QK^T scale) V (one head).

    The softmax gradient written out:

    * P = D^-1 A;
    * dV = P^T dO;
    * dP = dO V^T;
    * dS = P (dP - rowsum(P dP)), where rowsum(P dP)_i = dO_i . O_i;
    * dQ = scale dS K;
    * dK = scale dS^T Q.
    """
    Q, K, V, dO = _as64(Q), _as64(K), _as64(V), _as64(dO)
    n, d = Q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    S = (Q @ K.T) * scale
    if causal:
        i = np.arange(n)[:, None]
        j = np.arange(K.shape[0])[None, :]
        S = np.where(j <= i, S, -np.inf)
    c = S.max(axis=1, keepdims=True)
    A = np.exp(S - c)
    P = A / A.sum(axis=1, keepdims=True)
    dV = P.T @ dO
    dP = dO @ V.T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    return scale * dS @ K, scale * dS.T @ Q, dV


def _add_slots(dQ, dK, dV, Qr, Kr, Vr, qs, keys, dOr, lam, delta, w, u, scale):
    """Adds one group of slots to the gradients.

    Rows qs of the query side are given as Qr, dOr, lam (final lse) and
    delta. The key-slot side is given as keys (head-local key rows, repeats
    allowed), Kr, Vr, and the weights w (product) and u (row sum), each of
    shape [len(qs), len(keys)].
    """
    E = np.exp((Qr @ Kr.T) * scale - lam[:, None])
    ds = E * (w * (dOr @ Vr.T) - u * delta[:, None])
    dQ[qs] += scale * ds @ Kr
    np.add.at(dK, keys, scale * ds.T @ Qr)
    np.add.at(dV, keys, (w * E).T @ dOr)


def hyperattention_backward(Q, K, V, dO, *, causal, b, m, r=8, recursion_base=4096, seed=0,
                            G=None, head_ids=None):
    """dQ, dK, dV [H, n, d] (fp64) of sum(dO * O) for the HyperAttention output O.

    Arguments are those of hyperattention.hyperattention; the forward output,
    lse, buckets and sample lists are that function's.
    """
    H, n, d = np.shape(Q)
    scale = 1.0 / np.sqrt(d)
    art = {}
    O, lse = ha.hyperattention(Q, K, V, causal=causal, b=b, m=m, r=r,
                               recursion_base=recursion_base, seed=seed, artifacts=art,
                               G=G, head_ids=head_ids)
    dQ = np.zeros((H, n, d))
    dK = np.zeros((H, n, d))
    dV = np.zeros((H, n, np.shape(V)[2]))
    for h in range(H):
        Qh, Kh, Vh, dOh = _as64(Q[h]), _as64(K[h]), _as64(V[h]), _as64(dO[h])
        lam = lse[h]
        delta = (dOh * O[h]).sum(axis=1)
        # base cases: exact causal attention inside each diagonal block,
        # normalised by the final lse
        for lo, size in art["blocks"]:
            rows = np.arange(lo, lo + size)
            causal_w = (rows[None, :] <= rows[:, None]).astype(np.float64)
            _add_slots(dQ[h], dK[h], dV[h], Qh[rows], Kh[rows], Vh[rows], rows, rows,
                       dOh[rows], lam[rows], delta[rows], causal_w, causal_w, scale)
        for sub in art["sub"][h]:
            q_lo, k_lo, size, b_eff = sub["q_lo"], sub["k_lo"], sub["size"], sub["b_eff"]
            pq, pk = sub["perm_q"], sub["perm_k"]
            u_idx, v_idx = sub["u_idx"], sub["v_idx"]
            v_w = np.asarray(sub["v_w"], dtype=np.float64)
            for k in range(size // b_eff):
                qs = pq[k * b_eff:(k + 1) * b_eff]
                ks = pk[k * b_eff:(k + 1) * b_eff]
                one = np.ones((len(qs), len(ks)))
                _add_slots(dQ[h], dK[h], dV[h], Qh[qs], Kh[ks], Vh[ks], qs, ks, dOh[qs],
                           lam[qs], delta[qs], one, one, scale)
                # uniform sample: row sum only, outside the query's bucket
                keep_u = (sub["u_bucket"] != k).astype(np.float64)
                u = np.broadcast_to(sub["alpha"] * keep_u, (len(qs), len(u_idx)))
                _add_slots(dQ[h], dK[h], dV[h], Qh[qs], Kh[u_idx], Vh[u_idx], qs, u_idx,
                           dOh[qs], lam[qs], delta[qs], np.zeros_like(u), u, scale)
                # V-norm sample: product only, outside the query's bucket
                keep_v = (sub["v_bucket"] != k).astype(np.float64)
                w = np.broadcast_to(v_w * keep_v, (len(qs), len(v_idx)))
                _add_slots(dQ[h], dK[h], dV[h], Qh[qs], Kh[v_idx], Vh[v_idx], qs, v_idx,
                           dOh[qs], lam[qs], delta[qs], w, np.zeros_like(w), scale)
    return dQ, dK, dV


def hyperattention_backward_rows(Q, K, V, dO, q_rows, k_rows, *, causal, b, m, r=8,
                                 recursion_base=4096, seed=0, G=None, head_ids=None):
    """dQ at the query rows q_rows and dK, dV at the key rows k_rows, for
    every head, by the formulas of hyperattention_backward restricted to the
    slots those rows take part in (for problems too large to differentiate
    in full). The forward output is computed for the query rows that the
    requested gradients depend on.

    Returns dQ [H, len(q_rows), d], dK and dV [H, len(k_rows), d] (fp64).
    """
    H, n, d = np.shape(Q)
    scale = 1.0 / np.sqrt(d)
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    kw = dict(causal=causal, b=b, m=m, r=r, recursion_base=recursion_base, seed=seed, G=G,
              head_ids=head_ids)
    art = {}
    ha.hyperattention(Q, K, V, rows=np.zeros(0, dtype=np.int64), artifacts=art, **kw)
    dQ = np.zeros((H, len(q_rows), d))
    dK = np.zeros((H, len(k_rows), d))
    dV = np.zeros((H, len(k_rows), np.shape(V)[2]))
    for h in range(H):
        # query rows whose forward output the requested gradients need
        need = set(q_rows.tolist())
        for j in k_rows.tolist():
            for lo, size in art["blocks"]:
                if lo <= j < lo + size:
                    need.update(range(j, lo + size))
            for sub in art["sub"][h]:
                k_lo, size, b_eff = sub["k_lo"], sub["size"], sub["b_eff"]
                if not k_lo <= j < k_lo + size:
                    continue
                bk = sub["rank_k"][j - k_lo] // b_eff
                need.update(sub["perm_q"][bk * b_eff:(bk + 1) * b_eff].tolist())
                if j in sub["u_idx"] or j in sub["v_idx"]:
                    need.update(range(sub["q_lo"], sub["q_lo"] + size))
        rows = np.array(sorted(need), dtype=np.int64)
        hk = dict(kw)
        hk["head_ids"] = [h if head_ids is None else head_ids[h]]
        hk["G"] = None if G is None else G[h:h + 1]
        O, lse = ha.hyperattention(Q[h:h + 1], K[h:h + 1], V[h:h + 1], rows=rows, **hk)
        O, lam = O[0], lse[0]
        Qh, Kh, Vh, dOh = _as64(Q[h]), _as64(K[h]), _as64(V[h]), _as64(dO[h])
        delta = np.full(n, np.nan)
        delta[rows] = (dOh[rows] * O[rows]).sum(axis=1)

        def contrib(qs, keys, w, u):
            """(ds [len(qs), len(keys)], E) for query rows qs and key rows keys."""
            E = np.exp((Qh[qs] @ Kh[keys].T) * scale - lam[qs][:, None])
            ds = E * (w * (dOh[qs] @ Vh[keys].T) - u * delta[qs][:, None])
            return ds, E

        for t, i in enumerate(q_rows.tolist()):
            for lo, size in art["blocks"]:
                if lo <= i < lo + size:
                    keys = np.arange(lo, i + 1)
                    ds, _ = contrib([i], keys, 1.0, 1.0)
                    dQ[h, t] += scale * ds[0] @ Kh[keys]
            for sub in art["sub"][h]:
                q_lo, size, b_eff = sub["q_lo"], sub["size"], sub["b_eff"]
                if not q_lo <= i < q_lo + size:
                    continue
                pos = int(np.nonzero(sub["perm_q"] == i)[0][0])
                bk = pos // b_eff
                ks = sub["perm_k"][bk * b_eff:(bk + 1) * b_eff]
                ds, _ = contrib([i], ks, 1.0, 1.0)
                dQ[h, t] += scale * ds[0] @ Kh[ks]
                u = sub["alpha"] * (sub["u_bucket"] != bk)
                ds, _ = contrib([i], sub["u_idx"], 0.0, u[None, :])
                dQ[h, t] += scale * ds[0] @ Kh[sub["u_idx"]]
                wv = np.asarray(sub["v_w"], dtype=np.float64) * (sub["v_bucket"] != bk)
                ds, _ = contrib([i], sub["v_idx"], wv[None, :], 0.0)
                dQ[h, t] += scale * ds[0] @ Kh[sub["v_idx"]]

        for t, j in enumerate(k_rows.tolist()):
            for lo, size in art["blocks"]:
                if lo <= j < lo + size:
                    qs = np.arange(j, lo + size)
                    ds, E = contrib(qs, [j], 1.0, 1.0)
                    dK[h, t] += scale * ds[:, 0] @ Qh[qs]
                    dV[h, t] += E[:, 0] @ dOh[qs]
            for sub in art["sub"][h]:
                q_lo, k_lo, size, b_eff = sub["q_lo"], sub["k_lo"], sub["size"], sub["b_eff"]
                if not k_lo <= j < k_lo + size:
                    continue
                bk = sub["rank_k"][j - k_lo] // b_eff
                qs = sub["perm_q"][bk * b_eff:(bk + 1) * b_eff]
                ds, E = contrib(qs, [j], 1.0, 1.0)
                dK[h, t] += scale * ds[:, 0] @ Qh[qs]
                dV[h, t] += E[:, 0] @ dOh[qs]
                # sample slots drawn on row j: every query of the node outside
                # the slot's bucket
                allq = sub["perm_q"]
                qbk = np.arange(size) // b_eff
                for slot in np.nonzero(sub["u_idx"] == j)[0]:
                    keep = qbk != sub["u_bucket"][slot]
                    ds, _ = contrib(allq[keep], [j], 0.0, sub["alpha"])
                    dK[h, t] += scale * ds[:, 0] @ Qh[allq[keep]]
                for slot in np.nonzero(sub["v_idx"] == j)[0]:
                    keep = qbk != sub["v_bucket"][slot]
                    wv = float(sub["v_w"][slot])
                    ds, E = contrib(allq[keep], [j], wv, 0.0)
                    dK[h, t] += scale * ds[:, 0] @ Qh[allq[keep]]
                    dV[h, t] += wv * E[:, 0] @ dOh[allq[keep]]
    return dQ, dK, dV
