"""Hamming-sorted LSH and sortLSH buckets (test infrastructure only).

HA page, section "Algorithm": the first step finds the large entries of A by
hashing keys and queries into equal-size ("uniform-size") buckets with a
Hamming-sorted LSH (Definition 1, sortLSH), Algorithm 1 / Figure 1. The
result is a sparse mask M^H that is block-diagonal once Q and K are sorted.

The definition and the algorithm were lost in extraction. Readings taken:

* Hash family: r random Gaussian hyperplanes per head (the workloads name
  "r=8 Gaussian hyperplanes"), one set per head, shared by Q, K and every
  recursion level. Bit k of a row x is [<x, g_k> > 0] (zero maps to 0), and
  the r bits form c = sum_k bit_k 2^k.
* "Hamming-sorted": buckets are ordered by Gray-code rank, so that adjacent
  ranks differ in exactly one hyperplane sign. code(x) = the h with
  gray(h) = h XOR (h >> 1) equal to c.
* The sign is that of the fp64 sum of x_t * g_kt taken in the order
  t = 0 .. d-1 (every product of an fp32 or bf16 value with an fp32 value is
  exact in fp64, so this is a fully specified number).
* sortLSH: within one sub-problem, sort the query rows by (code, index) and
  the key rows by (code, index), stably; cut both sorted lists into chunks of
  b_eff = min(b, n_k) rows; query chunk k is paired with key chunk k.
* Hyperplanes are Gaussian via Box-Muller (Box and Muller, 1958) from two
  counter-based draws, evaluated as gaussian.py defines it (only IEEE-754
  binary64 basic operations, so any platform gets the same bits), rounded to
  fp32 and then to the nearest bfloat16 (ties to even), so that the product
  of a bf16 input with a hyperplane entry is exact in fp32. Element (k, t)
  of head h uses counters 2(k d + t) and 2(k d + t)+1 of purpose
  "hyperplane" with node 0.
"""

import numpy as np

from . import gaussian


def round_bf16(x32):
    """Nearest bfloat16 of an fp32 value (ties to even), returned as fp32."""
    bits = int(np.array(x32, dtype=np.float32).view(np.uint32))
    lsb = (bits >> 16) & 1
    bits = ((bits + 0x7FFF + lsb) >> 16) << 16
    return np.array(bits & 0xFFFFFFFF, dtype=np.uint32).view(np.float32)


def round_bf16_array(x32):
    """Nearest bfloat16 of each fp32 value (ties to even), returned as fp32."""
    bits = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bits = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    return (bits & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def hyperplanes(seed, heads, r, d):
    """G[h, k, t]: r Gaussian hyperplanes of dimension d per head (bf16 values
    held in fp32)."""
    a, b = gaussian.hyperplane_draws(seed, heads, r, d)
    g = gaussian.box_muller(a.ravel(), b.ravel()).astype(np.float32)
    return round_bf16_array(g).reshape(heads, r, d)


def projections_sequential(X, Gh):
    """p[i, k] = sum over t = 0..d-1, in that order, of X[i, t] * G[k, t] (fp64).

    Vectorised over rows and hyperplanes only; the sum over t runs one term at
    a time, so every entry is the left-to-right fp64 sum of exact products.
    """
    X = np.asarray(X, dtype=np.float64)
    G = np.asarray(Gh, dtype=np.float64)
    p = np.zeros((X.shape[0], G.shape[0]))
    for t in range(X.shape[1]):
        p = p + X[:, t:t + 1] * G[None, :, t]
    return p


def sign_bits(p):
    """c = sum_k [p_k > 0] 2^k, as int64."""
    r = p.shape[1]
    c = np.zeros(p.shape[0], dtype=np.int64)
    for k in range(r):
        c |= (p[:, k] > 0).astype(np.int64) << k
    return c


def gray(h):
    """Reflected binary Gray code of h."""
    return h ^ (h >> 1)


def gray_rank(c, r):
    """The h in [0, 2^r) whose Gray code is c.

    Bit k of h is the parity of bits k .. r-1 of c (read from the top bit
    down: the top bit is copied, each lower bit flips with every 1 above it).
    """
    c = np.asarray(c, dtype=np.int64)
    h = np.zeros_like(c)
    running = np.zeros_like(c)
    for k in range(r - 1, -1, -1):
        running = running ^ ((c >> k) & 1)
        h |= running << k
    return h


def hash_codes(X, Gh):
    """Definition 1 as read here: Gray rank of the hyperplane sign pattern."""
    r = np.asarray(Gh).shape[0]
    return gray_rank(sign_bits(projections_sequential(X, Gh)), r)


def sort_segment(codes):
    """Stable order of one segment by (code, index).

    Returns perm (sorted position -> local index) and rank (local index ->
    sorted position).
    """
    codes = np.asarray(codes)
    perm = np.argsort(codes, kind="stable").astype(np.int64)
    rank = np.empty_like(perm)
    rank[perm] = np.arange(len(perm))
    return perm, rank


def sortlsh(codes_q, codes_k, b):
    """Algorithm 1 (as read): equal-size buckets of sorted queries and keys.

    codes_q, codes_k: codes of the sub-problem's query rows and key rows
    (same length n_k). Returns a dict with perm/rank per side, b_eff, and the
    bucket of every query and key (rank // b_eff). Query bucket k attends to
    key bucket k: M^H_ij = [bucket_q(i) == bucket_k(j)].
    """
    n_k = len(codes_k)
    if len(codes_q) != n_k:
        raise ValueError("sortLSH expects equal numbers of queries and keys")
    b_eff = min(b, n_k)
    if n_k % b_eff:
        raise ValueError("bucket size must divide the sub-problem size")
    perm_q, rank_q = sort_segment(codes_q)
    perm_k, rank_k = sort_segment(codes_k)
    return {
        "b_eff": b_eff,
        "perm_q": perm_q, "rank_q": rank_q, "bucket_q": rank_q // b_eff,
        "perm_k": perm_k, "rank_k": rank_k, "bucket_k": rank_k // b_eff,
    }
