"""Pins for the oracle's random draws, hash and sortLSH (CPU only).

Each test checks the oracle against something other than itself: a published
known-answer vector, a brute-force definition, an exact rational computation,
or a textbook probability (SimHash collision rate).
"""

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import rng, sortlsh

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_known_answers():
    vals = [int(x, 16) for x in open(os.path.join(GOLDEN, "splitmix64_seed0.txt"))
            if x.strip() and not x.startswith("#")]
    state, out = 0, []
    for _ in vals:
        state, z = rng.splitmix64_next(state)
        out.append(z)
    assert out == vals
    # mix64 is the output for a given pre-step state
    assert rng.mix64(0) == vals[0]


def test_draw_fields_do_not_collide():
    seen = set()
    for p, h, node, t in itertools.product([1, 2, 3], [0, 1, 7], [0, 1, 5], range(40)):
        seen.add(rng.draw(123, p, h, node, t))
    assert len(seen) == 3 * 3 * 3 * 40
    with pytest.raises(ValueError):
        rng.pack(16, 0, 0, 0)
    with pytest.raises(ValueError):
        rng.pack(1, 0, 0, 1 << 24)


def test_draw_top_bits_uniform():
    # chi-square on the top 4 bits of 16000 draws, 15 dof: 99.99% bound ~ 44
    counts = np.zeros(16)
    for t in range(16000):
        counts[rng.draw(7, 2, 0, 1, t) >> 60] += 1
    chi2 = ((counts - 1000.0) ** 2 / 1000.0).sum()
    assert chi2 < 44


def test_gray_adjacent_ranks_differ_in_one_bit():
    for r in range(1, 9):
        for h in range(2 ** r - 1):
            assert bin(sortlsh.gray(h) ^ sortlsh.gray(h + 1)).count("1") == 1


def test_gray_rank_is_brute_force_inverse():
    for r in range(1, 9):
        table = {sortlsh.gray(h): h for h in range(2 ** r)}
        assert sorted(table) == list(range(2 ** r))
        c = np.arange(2 ** r)
        assert np.array_equal(sortlsh.gray_rank(c, r), [table[x] for x in c])


def test_hyperplane_gaussian_moments():
    G = sortlsh.hyperplanes(99, 4, 8, 64).astype(np.float64).ravel()   # 2048 values
    assert G.dtype == np.float64
    se = 1.0 / math.sqrt(G.size)
    assert abs(G.mean()) < 5 * se
    assert abs(G.var() - 1.0) < 5 * math.sqrt(2.0) * se
    from scipy import stats
    assert stats.kstest(G, "norm").pvalue > 1e-4


def test_hyperplanes_are_bf16_values():
    G = sortlsh.hyperplanes(3, 2, 8, 64)
    bits = G.view(np.uint32)
    assert not (bits & 0xFFFF).any()
    # rounding to nearest: the fp32 Gaussian is within half a bf16 ulp
    assert sortlsh.round_bf16(np.float32(1.0 + 2 ** -9)) == np.float32(1.0)
    assert sortlsh.round_bf16(np.float32(1.0 + 3 * 2 ** -9)) == np.float32(1.0 + 2 ** -7)


def test_hyperplanes_differ_by_head_and_seed():
    a = sortlsh.hyperplanes(1, 2, 2, 16)
    b = sortlsh.hyperplanes(2, 2, 2, 16)
    assert not np.array_equal(a[0], a[1])
    assert not np.array_equal(a, b)
    assert np.array_equal(a, sortlsh.hyperplanes(1, 2, 2, 16))


def test_sign_bits_follow_direction_of_hyperplane():
    G = sortlsh.hyperplanes(5, 1, 8, 64)[0]
    for k in range(8):
        c = sortlsh.sign_bits(sortlsh.projections_sequential(G[k:k + 1], G))
        assert (c[0] >> k) & 1 == 1
        c = sortlsh.sign_bits(sortlsh.projections_sequential(-G[k:k + 1], G))
        assert (c[0] >> k) & 1 == 0
    zero = np.zeros((1, 64))
    assert sortlsh.hash_codes(zero, G)[0] == 0


def test_sequential_projection_sign_matches_exact_rationals():
    rs = np.random.default_rng(0)
    G = sortlsh.hyperplanes(3, 1, 8, 32)[0]
    X = rs.standard_normal((40, 32)).astype(np.float32)
    p = sortlsh.projections_sequential(X, G)
    for i in range(40):
        for k in range(8):
            exact = sum(Fraction(float(X[i, t])) * Fraction(float(G[k, t]))
                        for t in range(32))
            assert (exact > 0) == (p[i, k] > 0)
            # the fp64 sequential sum is within the textbook bound of exact
            bound = 32 * 2.0 ** -53 * sum(abs(float(X[i, t]) * float(G[k, t]))
                                          for t in range(32))
            assert abs(float(exact) - p[i, k]) <= bound


def test_simhash_collision_rate():
    """P[bit agrees] = 1 - theta/pi for Gaussian hyperplanes (Charikar 2002)."""
    rs = np.random.default_rng(1)
    d = 64
    x = rs.standard_normal(d)
    u = rs.standard_normal(d)
    u -= (u @ x) / (x @ x) * x
    u /= np.linalg.norm(u)
    for theta in (0.3, 1.0, 2.0):
        y = np.linalg.norm(x) * (math.cos(theta) * x / np.linalg.norm(x)
                                 + math.sin(theta) * u)
        G = sortlsh.hyperplanes(11, 64, 8, d)          # 512 hyperplanes
        agree = 0
        for h in range(64):
            px = sortlsh.sign_bits(sortlsh.projections_sequential(x[None], G[h]))[0]
            py = sortlsh.sign_bits(sortlsh.projections_sequential(y[None], G[h]))[0]
            agree += 8 - bin(px ^ py).count("1")
        p = 1 - theta / math.pi
        se = math.sqrt(p * (1 - p) / 512)
        assert abs(agree / 512 - p) < 4 * se


def test_sort_segment_brute_force_rank():
    rs = np.random.default_rng(2)
    for n in (1, 7, 64, 100):
        codes = rs.integers(0, 5, n)
        perm, rank = sortlsh.sort_segment(codes)
        for i in range(n):
            brute = sum(1 for j in range(n) if (codes[j], j) < (codes[i], i))
            assert rank[i] == brute
        assert sorted(perm) == list(range(n))
        assert np.all(np.diff(codes[perm]) >= 0)
        for a, b in zip(perm[:-1], perm[1:]):
            if codes[a] == codes[b]:
                assert a < b


def test_sortlsh_buckets_equal_size_and_shape_errors():
    rs = np.random.default_rng(3)
    cq, ck = rs.integers(0, 256, 96), rs.integers(0, 256, 96)
    s = sortlsh.sortlsh(cq, ck, 32)
    assert s["b_eff"] == 32
    assert np.array_equal(np.bincount(s["bucket_q"]), [32] * 3)
    assert np.array_equal(np.bincount(s["bucket_k"]), [32] * 3)
    # keys in query i's bucket are exactly b_eff keys, chosen by sorted order
    i = int(np.argmin(cq))
    assert s["bucket_q"][i] == 0
    assert sortlsh.sortlsh(cq, ck, 500)["b_eff"] == 96
    with pytest.raises(ValueError):
        sortlsh.sortlsh(cq, ck, 40)
    with pytest.raises(ValueError):
        sortlsh.sortlsh(cq[:10], ck, 8)


def test_similar_rows_share_buckets():
    """A key equal to a query gets the same code, so with one bucket per code
    level they pair up (the property sortLSH exists for)."""
    rs = np.random.default_rng(4)
    G = sortlsh.hyperplanes(8, 1, 8, 64)[0]
    Q = rs.standard_normal((256, 64))
    assert np.array_equal(sortlsh.hash_codes(Q, G), sortlsh.hash_codes(Q * 3.0, G))


def test_zero_hyperplanes_give_the_local_block_mask():
    """r = 0 (a predefined mask in place of sortLSH): every code is 0, the
    stable sort keeps index order, and bucket k is rows [k b, (k + 1) b) on
    both sides (closed form)."""
    rs = np.random.default_rng(5)
    G = sortlsh.hyperplanes(3, 2, 0, 64)
    assert G.shape == (2, 0, 64)
    X = rs.standard_normal((96, 64))
    codes = sortlsh.hash_codes(X, G[1])
    assert np.array_equal(codes, np.zeros(96, dtype=codes.dtype))
    s = sortlsh.sortlsh(codes, sortlsh.hash_codes(X[::-1], G[0]), 32)
    idx = np.arange(96)
    assert np.array_equal(s["bucket_q"], idx // 32)
    assert np.array_equal(s["bucket_k"], idx // 32)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 128)])
def test_margin_rows_sit_where_asked(dtype, d):
    """The rows the GPU threshold test hashes: each projection on its chosen
    hyperplane is within 20% of c times the kernel's certainty margin, with
    the chosen sign, for c = 0.5, 1, 2, 10 (so both sides of the decision
    are exercised), and the oracle's bit follows that sign."""
    from tests.margin_rows import margin_set
    G, X, info = margin_set(21, d, dtype)
    assert len(X) >= 8 * 4 * 2 * 12
    k, c, ratio = info[:, 0].astype(int), info[:, 1], info[:, 2]
    assert np.all((np.abs(ratio) > 0.8 * c) & (np.abs(ratio) < 1.25 * c))
    bits = sortlsh.sign_bits(sortlsh.projections_sequential(X, G))
    assert np.array_equal((bits >> k) & 1, (ratio > 0).astype(int))
