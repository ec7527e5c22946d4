"""The seeded input generators (shared by both sides of every parity check)."""

import numpy as np

from approximate_softmax_attention_amd import workloads as wl


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -7 + 2 ** -9,
                  -2.5, 3.0e-39], dtype=np.float32)
    got = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(x))
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0);
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6 -> even (1 + 2^-6)
    assert list(got[:4]) == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7]
    assert got[4] == -2.5
    r = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    rb = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(r))
    assert np.all(np.abs(rb - r) <= np.abs(r) * 2 ** -8)


def test_rope_is_a_rotation_per_pair():
    X = np.random.default_rng(1).standard_normal((50, 16))
    Y = wl.rope(X)
    assert np.allclose(Y[0], X[0])
    n1 = X[:, :8] ** 2 + X[:, 8:] ** 2
    n2 = Y[:, :8] ** 2 + Y[:, 8:] ** 2
    assert np.allclose(n1, n2)
    # relative-position property: <rope(q)_p, rope(k)_p'> depends on p - p' only
    q, k = X[3], X[4]
    Qr = wl.rope(np.tile(q, (50, 1)))
    Kr = wl.rope(np.tile(k, (50, 1)))
    assert np.isclose(Qr[10] @ Kr[7], Qr[20] @ Kr[17])


def test_inputs_deterministic_and_planted():
    w = wl.scaled(wl.WORKLOADS["planted_noncausal_n8192_d64_h8_bf16"], n=256, heads=2)
    Q, K, V, pairs = wl.make_inputs(w)
    Q2, K2, V2, _ = wl.make_inputs(w)
    assert np.array_equal(Q, Q2) and np.array_equal(K, K2) and np.array_equal(V, V2)
    for h in range(2):
        p = pairs[h]
        assert len(p) > 0 and len(np.unique(p[:, 1])) == len(p)
        i, j = p[0]
        cos = Q[h, i] @ K[h, j] / np.linalg.norm(Q[h, i]) / np.linalg.norm(K[h, j])
        assert cos > 0.99
    # stored values are bf16-representable
    bits = wl.f32_to_bf16_bits(V)
    assert np.array_equal(wl.bf16_bits_to_f32(bits), V)


def test_make_inputs_large_is_deterministic_and_rounded():
    w = wl.scaled(wl.WORKLOADS["longctx_noncausal_n131072_d64_h8_bf16"], heads=2, n=1000)
    a = wl.make_inputs_large(w, chunk=256, workers=1)
    b = wl.make_inputs_large(w, chunk=256, workers=4)
    for x, y in zip(a, b):
        assert x.shape == (2, 1000, 64) and np.array_equal(x, y)
        # bf16 values: the low 16 bits of every fp32 pattern are zero
        assert not np.any(x.view(np.uint32) & 0xFFFF)
        assert abs(x.mean()) < 0.05 and abs(x.std() - 1) < 0.05
    # Q, K, V and the heads are different streams; chunks too
    assert not np.array_equal(a[0], a[1]) and not np.array_equal(a[0][0], a[0][1])
    assert not np.array_equal(a[0][0, :256], a[0][0, 256:512])
