"""HyperAttention forward pass, non-causal and causal (test infrastructure only).

HA page, section "Algorithm":

* Algorithm 1 (sortLSH) returns a sparse mask M^H of the large entries of A.
* Algorithm 2 (ApproxD) estimates the diagonal D from the entries under the
  mask plus a randomly chosen subset of the columns of A.
* Algorithm 3 (HyperAttention) combines that estimate with the product of
  the softmax matrix and V, sampled by the squared row norms of V.
* Figure 2 / Algorithm 4 (causal): M^C (.) A splits into two half-size causal
  diagonal blocks and the block A_21, which lies wholly below the diagonal and
  is unmasked; A_21 is handled by the non-causal algorithm and the diagonal
  blocks recursively. Section "Monkey-patching": the recursion stops at a
  small size, where attention is computed exactly; b = m = 256. Section
  "Single self-attention layer": the causal version splits Q, K, V and merges
  the attention outputs.

Readings taken where the page is silent (the listings were lost):

* Scores are s_ij = <q_i, k_j> / sqrt(d).
* For a sub-problem (query rows I, key rows J, n_k = |J| = |I|), with B(i) the
  keys in the bucket of query i (M^H restricted to row i), c_i the largest
  score row i evaluates, alpha and the uniform list l_t, the V-norm list j_t
  with weights w_t (see sampling.py):

      d~_i = sum_{j in B(i)} e^{s_ij - c_i}
             + alpha * sum_t [l_t not in B(i)] e^{s_il_t - c_i}
      N_i  = sum_{j in B(i)} e^{s_ij - c_i} V_j
             + sum_t w_t [j_t not in B(i)] e^{s_ij_t - c_i} V_{j_t}
      O_i  = N_i / d~_i,      lse_i = c_i + ln d~_i

  i.e. the masked part is exact and only the part outside M^H is sampled;
  so the result is exact attention whenever b or m covers the range.
* Causal recursion: a block [lo, lo + 2h) with node id kappa (the root is
  [0, n) with id 1) gives the off-diagonal sub-problem I = [lo + h, lo + 2h),
  J = [lo, lo + h) with node id kappa, and the diagonal blocks [lo, lo + h)
  (id 2 kappa) and [lo + h, lo + 2h) (id 2 kappa + 1). A block of size at most
  recursion_base is a base case: exact causal attention inside the block.
  An odd block size to be split is an error.
* Merge: each row's partial results over disjoint key sets are combined with
  exact.lse_merge.
* Non-causal: one sub-problem I = J = [0, n) with node id 1.
"""

import numpy as np

from . import exact, sampling, sortlsh


def schedule(n, causal, recursion_base):
    """Sub-problems [(level, node, q_lo, k_lo, size)] and base blocks [(lo, size)]."""
    if not causal:
        return [(1, 1, 0, 0, n)], []
    subs, blocks = [], []

    def split(lo, size, node, level):
        if size <= recursion_base:
            blocks.append((lo, size))
            return
        if size % 2:
            raise ValueError("odd block size in the causal recursion")
        h = size // 2
        subs.append((level, node, lo + h, lo, h))
        split(lo, h, 2 * node, level + 1)
        split(lo + h, h, 2 * node + 1, level + 1)

    split(0, n, 1, 1)
    return subs, blocks


def estimate_block(Qi, Kj, Vj, srt, u_idx, alpha, v_idx, v_w, scale,
                   want=None, with_product=True):
    """Algorithms 2 + 3 on one sub-problem (local indices).

    Qi, Kj, Vj: the sub-problem's query / key / value rows. srt: result of
    sortlsh.sortlsh. u_idx, v_idx: local key indices of the two samples.
    want: optional boolean mask over query rows to evaluate.
    Returns O (NaN rows where not wanted), lse, and d~ shifted by c (for
    rowsum_estimate when with_product is False).
    """
    n_k, dv = Qi.shape[0], Vj.shape[1]
    b_eff = srt["b_eff"]
    O = np.full((n_k, dv), np.nan)
    lse = np.full(n_k, np.nan)
    bk = srt["bucket_k"]
    for k in range(n_k // b_eff):
        qs = srt["perm_q"][k * b_eff:(k + 1) * b_eff]
        if want is not None:
            qs = qs[want[qs]]
            if len(qs) == 0:
                continue
        ks = srt["perm_k"][k * b_eff:(k + 1) * b_eff]
        S_b = (Qi[qs] @ Kj[ks].T) * scale
        S_u = (Qi[qs] @ Kj[u_idx].T) * scale
        keep_u = (bk[u_idx] != k).astype(np.float64)
        cols = [S_b, S_u]
        if with_product:
            S_v = (Qi[qs] @ Kj[v_idx].T) * scale
            keep_v = (bk[v_idx] != k).astype(np.float64)
            cols.append(S_v)
        c = np.max(np.concatenate(cols, axis=1), axis=1, keepdims=True)
        E_b = np.exp(S_b - c)
        dt = E_b.sum(axis=1) + alpha * (keep_u * np.exp(S_u - c)).sum(axis=1)
        lse[qs] = c[:, 0] + np.log(dt)
        if with_product:
            coef_v = np.asarray(v_w, dtype=np.float64) * keep_v
            N = E_b @ Vj[ks] + (coef_v * np.exp(S_v - c)) @ Vj[v_idx]
            O[qs] = N / dt[:, None]
    return O, lse


def _head_inputs(Q, K, V):
    return (np.asarray(Q, dtype=np.float64), np.asarray(K, dtype=np.float64),
            np.asarray(V, dtype=np.float64))


def hyperattention(Q, K, V, *, causal, b, m, r=8, recursion_base=4096, seed=0,
                   rows=None, artifacts=None, G=None, head_ids=None, sample_from=None):
    """HyperAttention forward for all heads. Q, K, V: [H, n, d].

    rows: optional list of query rows to evaluate (all heads); others are NaN.
    artifacts: optional dict filled with codes, sorts and sample lists.
    G: optional hyperplanes [H, r, d] (defaults to sortlsh.hyperplanes(seed)).
    head_ids: the head index of each entry of the first axis (default 0..H-1);
    hyperplanes and random draws depend on it.
    sample_from: optional (Q', K', V') of the same shapes: the hash codes come
    from Q', K' and the V-norm weights from V' instead of the inputs, so the
    buckets and sample lists stay fixed while the inputs move (the estimator
    as a function of Q, K, V for a fixed draw, whose derivative the backward
    pass computes).
    Returns O [H, n, d] and lse [H, n] (fp64).
    """
    H, n, d = np.shape(Q)
    scale = 1.0 / np.sqrt(d)
    hids = list(range(H)) if head_ids is None else list(head_ids)
    if G is None:
        G = sortlsh.hyperplanes(seed, max(hids) + 1, r, d)[hids]
    subs, blocks = schedule(n, causal, recursion_base)
    want = None
    if rows is not None:
        want = np.zeros(n, dtype=bool)
        want[np.asarray(rows)] = True
    O_all = np.full((H, n, np.shape(V)[2]), np.nan)
    lse_all = np.full((H, n), np.nan)
    if artifacts is not None:
        artifacts.update(G=G, codes_q=[], codes_k=[], W=[], P=[], subs=subs,
                         blocks=blocks, sub=[])
    for h in range(H):
        hid = hids[h]
        Qh, Kh, Vh = _head_inputs(Q[h], K[h], V[h])
        Qs, Ks, Vs = (Qh, Kh, Vh) if sample_from is None else _head_inputs(
            sample_from[0][h], sample_from[1][h], sample_from[2][h])
        codes_q = sortlsh.hash_codes(Qs, G[h])
        codes_k = sortlsh.hash_codes(Ks, G[h])
        _, W, P = sampling.vnorm_weights(Vs)
        head_art = []
        O = np.full((n, Vh.shape[1]), np.nan)
        lse = np.full(n, np.nan)
        # base cases: exact causal attention inside each diagonal block
        for lo, size in blocks:
            sl = slice(lo, lo + size)
            if want is None:
                O[sl], lse[sl] = exact.exact_attention(Qh[sl], Kh[sl], Vh[sl],
                                                       causal=True, scale=scale)
            elif want[sl].any():
                loc = np.nonzero(want[sl])[0]
                O[lo + loc], lse[lo + loc] = exact.exact_attention_rows(
                    Qh[sl], Kh[sl], Vh[sl], loc, causal=True, scale=scale)
        for level, node, q_lo, k_lo, size in subs:
            I = slice(q_lo, q_lo + size)
            J = slice(k_lo, k_lo + size)
            srt = sortlsh.sortlsh(codes_q[I], codes_k[J], b)
            u_idx, alpha = sampling.uniform_samples(seed, hid, node, k_lo, size, m)
            v_idx, v_w = sampling.vnorm_samples(seed, hid, node, k_lo, size, P, W, m)
            w_sub = None if want is None else want[I]
            if w_sub is None or w_sub.any():
                Op, lp = estimate_block(Qh[I], Kh[J], Vh[J], srt, u_idx - k_lo,
                                        alpha, v_idx - k_lo, v_w, scale, want=w_sub)
                if causal:
                    sel = ~np.isnan(lp)
                    rows_i = np.arange(q_lo, q_lo + size)[sel]
                    O[rows_i], lse[rows_i] = exact.lse_merge(
                        [(O[rows_i], lse[rows_i]), (Op[sel], lp[sel])])
                else:
                    O[I], lse[I] = Op, lp
            if artifacts is not None:
                head_art.append(dict(level=level, node=node, q_lo=q_lo, k_lo=k_lo,
                                     size=size, b_eff=srt["b_eff"],
                                     perm_q=srt["perm_q"] + q_lo,
                                     perm_k=srt["perm_k"] + k_lo,
                                     rank_k=srt["rank_k"],
                                     u_idx=u_idx, alpha=alpha,
                                     u_bucket=srt["bucket_k"][u_idx - k_lo],
                                     v_idx=v_idx, v_w=v_w,
                                     v_bucket=srt["bucket_k"][v_idx - k_lo]))
        O_all[h], lse_all[h] = O, lse
        if artifacts is not None:
            artifacts["codes_q"].append(codes_q)
            artifacts["codes_k"].append(codes_k)
            artifacts["W"].append(W)
            artifacts["P"].append(P)
            artifacts["sub"].append(head_art)
    return O_all, lse_all


def rowsum_estimate(Q, K, *, b, m, r=8, seed=0, G=None):
    """Algorithm 2 alone, non-causal: log d~_i per row (lse without the product).

    Returns lse [H, n] = c_i + ln d~_i with d~ as in estimate_block.
    """
    H, n, d = np.shape(Q)
    scale = 1.0 / np.sqrt(d)
    if G is None:
        G = sortlsh.hyperplanes(seed, H, r, d)
    out = np.empty((H, n))
    for h in range(H):
        Qh = np.asarray(Q[h], dtype=np.float64)
        Kh = np.asarray(K[h], dtype=np.float64)
        srt = sortlsh.sortlsh(sortlsh.hash_codes(Qh, G[h]),
                              sortlsh.hash_codes(Kh, G[h]), b)
        u_idx, alpha = sampling.uniform_samples(seed, h, 1, 0, n, m)
        _, lse = estimate_block(Qh, Kh, Kh[:, :1], srt, u_idx, alpha,
                                np.zeros(0, dtype=np.int64), np.zeros(0), scale,
                                with_product=False)
        out[h] = lse
    return out
