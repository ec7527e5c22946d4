"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Integer artefacts (hash codes, V-norm weights and prefix sums, sortLSH
permutations and ranks, sample lists) must be bit-exact; O and lse must be
within the max-relative tolerance of gpu_util.TOL. Inputs come from the shared
seeded generators in approximate_softmax_attention_amd.workloads.
"""

import numpy as np
import pytest

from approximate_softmax_attention_amd import workloads as wl
from oracle import exact as oexact
from oracle import hyperattention as oha
from oracle import sortlsh as osl
from tests.gpu_util import (TOL, banner, check_artifacts, max_rel, region, run_forward,
                            to_dev, to_np)

pytestmark = pytest.mark.gpu


def _api():
    from approximate_softmax_attention_amd import api
    return api


def _inputs(name, **changes):
    w = wl.scaled(wl.WORKLOADS[name], **changes) if changes else wl.WORKLOADS[name]
    Q, K, V, pairs = wl.make_inputs(w)
    return w, Q, K, V, pairs


def _sync():
    import torch
    torch.cuda.synchronize()


# ------------------------------------------------------------ exact attention

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 77, 300, 5000])
def test_exact_attention(dtype, d, causal, n):
    banner(f"exact dtype={dtype} d={d} causal={causal} n={n}")
    w, Q, K, V, _ = _inputs("single_head_noncausal_n1024_d64_fp32", heads=2, n=n, d=d,
                            dtype=dtype)
    api = _api()
    O, L = api.exact(to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype), causal=causal,
                     return_lse=True)
    _sync()
    ref = [oexact.exact_attention(Q[h], K[h], V[h], causal=causal) for h in range(2)]
    Oref = np.stack([r[0] for r in ref])
    Lref = np.stack([r[1] for r in ref])
    assert max_rel(to_np(O), Oref) <= TOL[dtype]
    assert np.abs(to_np(L) - Lref).max() <= TOL[dtype]


# ----------------------------------------------------------------- the hash

@pytest.mark.parametrize("dtype,d", [("fp32", 64), ("bf16", 64), ("bf16", 128), ("fp32", 128)])
def test_sortlsh_hash_bit_exact(dtype, d):
    banner(f"hash dtype={dtype} d={d}")
    w, Q, K, V, _ = _inputs("single_head_noncausal_n1024_d64_fp32", heads=3, n=4099, d=d,
                            dtype=dtype)
    Q[0, 5] = 0.0                      # a zero row hashes to code 0
    api = _api()
    for r in (1, 5, 8):
        codes, perm = api.sortlsh_hash(to_dev(Q, dtype), r=r, seed=31, with_perm=True)
        _sync()
        G = osl.hyperplanes(31, 3, r, d)
        for h in range(3):
            ref = osl.hash_codes(Q[h], G[h])
            assert np.array_equal(codes[h].cpu().numpy(), ref)
            rp, _ = osl.sort_segment(ref)
            assert np.array_equal(perm[h].cpu().numpy(), rp)
        assert codes[0, 5].item() == 0


def test_sortlsh_sort_spans_several_chunks():
    """n = 10007 rows per head: the stable sort runs over three chunks (two
    whole ones and a ragged tail), so each chunk's offsets come from its
    segment's earlier chunk histograms."""
    banner("hash + sort n=10007")
    w, Q, K, V, _ = _inputs("single_head_noncausal_n1024_d64_fp32", heads=2, n=10007, d=128,
                            dtype="bf16")
    api = _api()
    codes, perm = api.sortlsh_hash(to_dev(Q, "bf16"), r=8, seed=77, with_perm=True)
    _sync()
    G = osl.hyperplanes(77, 2, 8, 128)
    for h in range(2):
        ref = osl.hash_codes(Q[h], G[h])
        assert np.array_equal(codes[h].cpu().numpy(), ref)
        rp, _ = osl.sort_segment(ref)
        assert np.array_equal(perm[h].cpu().numpy(), rp)


def test_hash_without_hyperplanes_is_the_identity_order():
    """r = 0: every code is 0 and the stable sort keeps index order (ragged
    n, so the code rows of the second head are not 16-byte aligned)."""
    banner("hash r=0")
    import torch
    api = _api()
    x = torch.randn((3, 1003, 64), device="cuda", dtype=torch.bfloat16)
    codes, perm = api.sortlsh_hash(x, r=0, seed=5, with_perm=True)
    _sync()
    assert int(codes.abs().sum()) == 0
    ident = torch.arange(1003, device="cuda", dtype=torch.int32).expand(3, -1)
    assert torch.equal(perm, ident)


def test_hash_near_zero_projections_use_exact_sign():
    """Rows almost orthogonal to a hyperplane exercise the fp64 re-check."""
    banner("hash near-zero")
    d, H = 64, 1
    G = osl.hyperplanes(5, H, 8, d)[0].astype(np.float64)
    rs = np.random.default_rng(0)
    X = rs.standard_normal((512, d))
    for i in range(512):                         # project out hyperplane i % 8
        g = G[i % 8]
        X[i] -= (X[i] @ g) / (g @ g) * g
        X[i] += rs.standard_normal() * 1e-7 * g   # tiny signed residue
    X = X.astype(np.float32)[None]
    api = _api()
    codes = api.sortlsh_hash(to_dev(X, "fp32"), r=8, seed=5)
    _sync()
    ref = osl.hash_codes(X[0], osl.hyperplanes(5, H, 8, d)[0])
    assert np.array_equal(codes[0].cpu().numpy(), ref)


def test_hash_bf16_cancelling_rows_use_exact_sign():
    """bf16 rows built so that <x, g_k> is exactly 0 or a tiny fraction of
    sum |x_t g_kt> (far below the fp32 certainty bound) must take the fp64
    re-check and agree with the sequential definition."""
    banner("hash bf16 cancellation")
    d, r = 128, 8
    G = osl.hyperplanes(17, 1, r, d)[0]
    rs = np.random.default_rng(3)
    X = np.zeros((512, d), dtype=np.float32)
    for i in range(512):
        k = i % r
        a, b, c = rs.choice(d, 3, replace=False)
        X[i, a], X[i, b] = G[k, b], -G[k, a]            # cancels exactly on g_k
        if i % 3:
            X[i, c] = np.float32(2.0 ** -30) * (1 if i % 2 else -1)
        X[i] += 0.0
    api = _api()
    codes = api.sortlsh_hash(to_dev(X[None], "bf16"), r=r, seed=17)
    _sync()
    ref = osl.hash_codes(X, G)
    assert np.array_equal(codes[0].cpu().numpy(), ref)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 128), ("fp32", 64)])
def test_hash_rows_at_the_certainty_margin(dtype, d):
    """Rows whose projection on one hyperplane sits at 0.5, 1, 2 and 10 times
    the kernel's certainty margin (3 gamma_d sum |x_t g_t| on the bf16 MFMA
    path, 4 gamma_d |x| |g| on the fp32 path), both signs, every hyperplane:
    codes bit-exact against the fp64 sequential definition, whichever side
    of the margin the fp32 value falls."""
    banner(f"hash at the certainty margin {dtype} d={d}")
    from tests.margin_rows import margin_set
    G, X, info = margin_set(21, d, dtype)
    api = _api()
    codes = api.sortlsh_hash(to_dev(X[None].astype(np.float32), dtype), r=8, seed=21)
    _sync()
    ref = osl.hash_codes(X, G)
    got = codes[0].cpu().numpy()
    bad = np.nonzero(got != ref)[0]
    assert len(bad) == 0, [(int(i), info[i].tolist()) for i in bad[:8]]
    print(f"{len(X)} rows at 0.5/1/2/10 x the margin: codes bit-exact", flush=True)


# ------------------------------------------------- forward: integer artefacts

def _check_artifacts(w, Q, K, V, ws, layout, art):
    check_artifacts(w, ws, layout, art, list(range(w.heads)))


def _run_forward(w, Q, K, V):
    return run_forward(w, Q, K, V)


FORWARD_CASES = {
    # name: (workload, changes)
    "c1_full": ("single_head_noncausal_n1024_d64_fp32", {}),
    "noncausal_bf16_d128_ragged_bucket": ("single_head_noncausal_n1024_d64_fp32",
                                          dict(heads=2, n=1000, d=128, dtype="bf16", b=100,
                                               m=37)),
    "causal_fp32_d64": ("chatglm2_causal_n32768_d128_h32_bf16",
                        dict(heads=2, n=2048, d=64, dtype="fp32", b=64, m=48,
                             recursion_base=256)),
    "causal_bf16_d128": ("chatglm2_causal_n32768_d128_h32_bf16",
                         dict(heads=2, n=4096, b=128, m=100, recursion_base=512)),
    "causal_bf16_ragged_base": ("chatglm2_causal_n32768_d128_h32_bf16",
                                dict(heads=1, n=1536, b=96, m=300, recursion_base=200)),
    # fp32 at d = 128: 64-key fp32 tiles (16 per slot window), causal with
    # recursion and merge, and non-causal
    "causal_fp32_d128": ("chatglm2_causal_n32768_d128_h32_bf16",
                         dict(heads=2, n=2048, dtype="fp32", b=64, m=48, recursion_base=256)),
    "noncausal_fp32_d128": ("single_head_noncausal_n1024_d64_fp32",
                            dict(heads=2, n=1024, d=128, b=128, m=96)),
    # bf16 items of more than 8 tiles (b + 2m > 1024 slots): the slot window
    # is refilled inside the item
    "noncausal_bf16_d128_slot_refill": ("single_head_noncausal_n1024_d64_fp32",
                                        dict(heads=2, n=4096, d=128, dtype="bf16", b=512,
                                             m=512)),
    "noncausal_bf16_d64_slot_refill": ("single_head_noncausal_n1024_d64_fp32",
                                       dict(heads=2, n=4096, dtype="bf16", b=256, m=512)),
    "causal_bf16_d128_slot_refill": ("chatglm2_causal_n32768_d128_h32_bf16",
                                     dict(heads=1, n=8192, b=512, m=300, recursion_base=1024)),
    # a segment of 9000 rows: three sort chunks, the last ragged
    "noncausal_bf16_d64_three_sort_chunks": ("single_head_noncausal_n1024_d64_fp32",
                                             dict(heads=2, n=9000, dtype="bf16", b=120, m=100)),
    # r = 0: the local block mask in place of sortLSH
    "local_mask_causal_bf16_d128": ("chatglm2_causal_n32768_d128_h32_bf16",
                                    dict(heads=2, n=4096, b=128, m=100, r=0,
                                         recursion_base=512)),
    "local_mask_noncausal_fp32_d64": ("single_head_noncausal_n1024_d64_fp32",
                                      dict(heads=2, n=1024, b=64, m=48, r=0)),
}


@pytest.mark.parametrize("case", sorted(FORWARD_CASES))
def test_forward_matches_oracle(case):
    name, changes = FORWARD_CASES[case]
    banner(f"forward {case}")
    w, Q, K, V, _ = _inputs(name, **changes)
    O, L, ws, layout = _run_forward(w, Q, K, V)
    art = {}
    Oref, Lref = oha.hyperattention(Q, K, V, causal=w.causal, b=w.b, m=w.m, r=w.r,
                                    recursion_base=w.recursion_base, seed=w.method_seed,
                                    artifacts=art)
    _check_artifacts(w, Q, K, V, ws, layout, art)
    assert max_rel(to_np(O), Oref) <= TOL[w.dtype]
    assert np.abs(to_np(L) - Lref).max() <= TOL[w.dtype]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_forward_empty_vnorm_lists(dtype):
    """V zero on the first half of the keys: every sub-problem whose key range
    lies there has V-norm total 0, so its V-norm list is empty (the product
    keeps only the bucket term), while the others sample as usual."""
    banner(f"forward empty V-norm lists {dtype}")
    w, Q, K, V, _ = _inputs("chatglm2_causal_n32768_d128_h32_bf16", heads=2, n=2048, d=64,
                            dtype=dtype, b=64, m=48, recursion_base=256)
    V = V.copy()
    V[0, : w.n // 2] = 0.0
    V[1, : w.n // 4] = 0.0
    O, L, ws, layout = _run_forward(w, Q, K, V)
    art = {}
    Oref, Lref = oha.hyperattention(Q, K, V, causal=True, b=w.b, m=w.m, r=w.r,
                                    recursion_base=w.recursion_base, seed=w.method_seed,
                                    artifacts=art)
    _check_artifacts(w, Q, K, V, ws, layout, art)
    assert max_rel(to_np(O), Oref) <= TOL[w.dtype]
    assert np.abs(to_np(L) - Lref).max() <= TOL[w.dtype]


ROPE_CASES = {
    # name: (workload, changes); inputs are the workload's rows before RoPE
    "causal_bf16_d128_fused": ("chatglm2_causal_n32768_d128_h32_bf16",
                               dict(heads=2, n=4096, b=128, m=100, recursion_base=512,
                                    rope=False)),
    "noncausal_fp32_d64": ("single_head_noncausal_n1024_d64_fp32",
                           dict(heads=2, n=1024, b=64, m=48)),
    "causal_bf16_d64_local_mask": ("chatglm2_causal_n32768_d128_h32_bf16",
                                   dict(heads=2, n=2048, d=64, b=64, m=48, r=0,
                                        recursion_base=256, rope=False)),
    "causal_bf16_no_recursion": ("chatglm2_causal_n32768_d128_h32_bf16",
                                 dict(heads=2, n=512, b=128, m=64, recursion_base=4096,
                                      rope=False)),
}


@pytest.mark.parametrize("case", sorted(ROPE_CASES))
def test_forward_rope_matches_oracle(case):
    """Rotary embedding on the device (fused with the hash for bf16): the
    rotated rows are bit-exact, then every artefact and output as in the
    plain forward on those rows."""
    from oracle import rope as orope
    import torch
    name, changes = ROPE_CASES[case]
    banner(f"forward rope {case}")
    w, Q, K, V, _ = _inputs(name, **changes)
    api = _api()
    dt = w.dtype
    q, k, v = (to_dev(x, dt) for x in (Q, K, V))
    kw = dict(causal=w.causal, b=w.b, m=w.m, r=w.r, recursion_base=w.recursion_base,
              dtype=api.HA_BF16 if dt == "bf16" else api.HA_F32)
    layout = api.workspace_layout(w.n, w.d, w.heads, **kw)
    ws = api.alloc_workspace(api.workspace_bytes(w.n, w.d, w.heads, **kw), "cuda")
    ws.fill_(0xFF)
    O, L, Qr, Kr = api.forward_rope(q, k, v, causal=w.causal, b=w.b, m=w.m, r=w.r,
                                    recursion_base=w.recursion_base, seed=w.method_seed,
                                    return_lse=True, return_rotated=True, workspace=ws)
    _sync()
    tab = orope.angle_table(w.n, w.d, 10000.0)
    Qo = np.stack([orope.rope(Q[h], dtype=dt, table=tab) for h in range(w.heads)])
    Ko = np.stack([orope.rope(K[h], dtype=dt, table=tab) for h in range(w.heads)])
    assert np.array_equal(to_np(Qr), Qo) and np.array_equal(to_np(Kr), Ko)
    art = {}
    Oref, Lref = oha.hyperattention(Qo, Ko, V, causal=w.causal, b=w.b, m=w.m, r=w.r,
                                    recursion_base=w.recursion_base, seed=w.method_seed,
                                    artifacts=art)
    if not (w.causal and w.n <= w.recursion_base):
        _check_artifacts(w, Qo, Ko, V, ws, layout, art)
    assert max_rel(to_np(O), Oref) <= TOL[w.dtype]
    assert np.abs(to_np(L) - Lref).max() <= TOL[w.dtype]


def test_planted_workload_full():
    """8 heads, n = 8192, d = 64, bf16, planted heavy keys: full parity."""
    banner("forward planted n=8192")
    w, Q, K, V, pairs = _inputs("planted_noncausal_n8192_d64_h8_bf16")
    O, L, ws, layout = _run_forward(w, Q, K, V)
    art = {}
    Oref, Lref = oha.hyperattention(Q, K, V, causal=False, b=w.b, m=w.m, r=w.r,
                                    seed=w.method_seed, artifacts=art)
    _check_artifacts(w, Q, K, V, ws, layout, art)
    assert max_rel(to_np(O), Oref) <= TOL["bf16"]
    assert np.abs(to_np(L) - Lref).max() <= TOL["bf16"]
    # planted recall (reported): fraction of planted pairs sharing a bucket
    hits = tot = 0
    for h in range(w.heads):
        a = art["sub"][h][0]
        bq = np.empty(w.n, dtype=np.int64)
        bq[a["perm_q"]] = np.arange(w.n) // a["b_eff"]
        bk = np.empty(w.n, dtype=np.int64)
        bk[a["perm_k"]] = np.arange(w.n) // a["b_eff"]
        p = pairs[h]
        hits += int((bq[p[:, 0]] == bk[p[:, 1]]).sum())
        tot += len(p)
    print(f"planted recall {hits / tot:.3f} over {tot} pairs")
    assert hits / tot > 0.5


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 128), ("fp32", 64)])
def test_rowsum_estimate_matches_oracle(dtype, d):
    banner(f"rowsum {dtype} d={d}")
    w, Q, K, V, _ = _inputs("single_head_noncausal_n1024_d64_fp32", heads=2, n=2048, d=d,
                            dtype=dtype, b=128, m=96)
    api = _api()
    ld = api.rowsum_estimate(to_dev(Q, dtype), to_dev(K, dtype), b=w.b, m=w.m, r=w.r,
                             seed=w.method_seed)
    _sync()
    ref = oha.rowsum_estimate(Q, K, b=w.b, m=w.m, r=w.r, seed=w.method_seed)
    assert np.abs(to_np(ld) - ref).max() <= TOL[dtype]


# ---------------------------------------------------------------- edge cases

def test_reductions_to_exact_on_gpu():
    banner("reductions")
    api = _api()
    w, Q, K, V, _ = _inputs("single_head_noncausal_n1024_d64_fp32", heads=2, n=512, d=64)
    q, k, v = (to_dev(x, "fp32") for x in (Q, K, V))
    Oe = np.stack([oexact.exact_attention(Q[h], K[h], V[h])[0] for h in range(2)])
    Oc = np.stack([oexact.exact_attention(Q[h], K[h], V[h], causal=True)[0] for h in range(2)])
    O1 = api.forward(q, k, v, causal=False, b=512, m=5, seed=3)       # one bucket
    O2 = api.forward(q, k, v, causal=False, b=16, m=512, seed=3)      # exhaustive samples
    O3 = api.forward(q, k, v, causal=True, b=256, m=3, recursion_base=64, seed=3)
    O4 = api.forward(q, k, v, causal=True, b=8, m=2, recursion_base=512, seed=3)
    _sync()
    assert max_rel(to_np(O1), Oe) <= 1e-3
    assert max_rel(to_np(O2), Oe) <= 1e-3
    assert max_rel(to_np(O3), Oc) <= 1e-3
    assert max_rel(to_np(O4), Oc) <= 1e-3


def test_empty_and_error_paths():
    banner("edge")
    import torch
    api = _api()
    from approximate_softmax_attention_amd._lib import HyperAttnError
    z = torch.empty((2, 0, 64), device="cuda", dtype=torch.bfloat16)
    assert api.forward(z, z, z, causal=True).shape == (2, 0, 64)
    assert api.exact(z, z, z).shape == (2, 0, 64)
    q = torch.randn((1, 96, 64), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(HyperAttnError, match="HA_ERR_SHAPE"):
        api.forward(q, q, q, causal=False, b=40, m=8)              # 40 does not divide 96
    with pytest.raises(HyperAttnError, match="HA_ERR_SHAPE"):
        api.forward(q, q, q, causal=True, b=1, m=8, recursion_base=2)   # 96->...->6->3: 3 > 2 is odd
    q3 = torch.randn((1, 96, 32), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(HyperAttnError, match="HA_ERR_UNSUPPORTED"):
        api.exact(q3, q3, q3)
    # caller buffers of the wrong size or type are refused before any launch
    q = torch.randn((1, 128, 64), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out"):
        api.forward(q, q, q, causal=False, b=64, m=32, out=torch.empty_like(q)[:, :64])
    with pytest.raises(ValueError, match="lse_out"):
        api.exact(q, q, q, return_lse=True,
                  lse_out=torch.empty((1, 64), device="cuda", dtype=torch.float32))
    with pytest.raises(ValueError, match="workspace"):
        api.forward(q, q, q, causal=False, b=64, m=32,
                    workspace=torch.empty(1 << 20, device="cuda", dtype=torch.float32))
    # a workspace one byte short is refused by the library itself
    nb = api.workspace_bytes(128, 64, 1, causal=False, b=64, m=32)
    with pytest.raises(HyperAttnError):
        api.forward(q, q, q, causal=False, b=64, m=32,
                    workspace=torch.empty(nb - 1, device="cuda", dtype=torch.uint8))


def test_deterministic_repeat():
    banner("determinism")
    import torch
    api = _api()
    w, Q, K, V, _ = _inputs("chatglm2_causal_n32768_d128_h32_bf16", heads=2, n=4096, b=128,
                            m=128, recursion_base=512)
    q, k, v = (to_dev(x, "bf16") for x in (Q, K, V))
    a = api.forward(q, k, v, causal=True, b=128, m=128, recursion_base=512, seed=9)
    b = api.forward(q, k, v, causal=True, b=128, m=128, recursion_base=512, seed=9)
    c = api.forward(q, k, v, causal=True, b=128, m=128, recursion_base=512, seed=10)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert not torch.equal(a, c)


def test_fresh_seed_every_call():
    """Every call draws its hyperplanes on the device from its own seed, into
    its own workspace, on the call's stream: twenty seeds enqueued back to
    back without a wait each give the codes of their own seed, O and lse match
    the oracle, and a repeat call gives the same bytes."""
    banner("hyperplanes drawn per call: 20 seeds back to back")
    import torch
    api = _api()
    w, Q, K, V, _ = _inputs("planted_noncausal_n8192_d64_h8_bf16", heads=2, n=1024, b=128, m=64,
                            planted=0)
    q, k, v = (to_dev(x, "bf16") for x in (Q, K, V))
    kw = dict(causal=False, b=w.b, m=w.m, r=w.r)
    layout = api.workspace_layout(w.n, w.d, w.heads, **kw)
    nb = api.workspace_bytes(w.n, w.d, w.heads, **kw)
    seeds = list(range(7000, 7020))
    outs = {}
    for sd in seeds:
        ws = api.alloc_workspace(nb, "cuda")
        ws.fill_(0xAB)
        o, lse = api.forward(q, k, v, seed=sd, return_lse=True, workspace=ws, **kw)
        outs[sd] = (o, lse, ws)
    _sync()
    for sd in seeds:
        cq = region(outs[sd][2], layout, "CODES_Q", np.uint8).reshape(w.heads, w.n)
        G = osl.hyperplanes(sd, w.heads, w.r, w.d)
        for h in range(w.heads):
            assert np.array_equal(cq[h], osl.hash_codes(Q[h], G[h])), (sd, h)
    sd = seeds[-1]
    Oref, Lref = oha.hyperattention(Q, K, V, seed=sd, **kw)
    assert max_rel(to_np(outs[sd][0]), Oref) <= TOL["bf16"]
    assert np.abs(to_np(outs[sd][1]) - Lref).max() <= TOL["bf16"]
    again = api.forward(q, k, v, seed=sd, **kw)
    _sync()
    assert torch.equal(again, outs[sd][0])


@pytest.mark.parametrize("d,r", [(128, 8), (64, 8), (128, 3)])
def test_device_hyperplanes_equal_oracle(d, r):
    """The hyperplanes the device draws into the workspace (fp32 values and
    the bf16 layout with rows r..15 zero) equal the oracle's bit for bit, for
    64 heads and three seeds (the binary64 Box-Muller is evaluated with the
    same correctly rounded operations on both sides)."""
    banner(f"device hyperplanes d={d} r={r}")
    import torch
    api = _api()
    H, n = 64, 256
    x = torch.randn((H, n, d), device="cuda", dtype=torch.bfloat16)
    kw = dict(causal=False, b=128, m=64, r=r)
    layout = api.workspace_layout(n, d, H, **kw)
    for sd in (0, 1004, 2 ** 63 + 12345):
        ws = api.alloc_workspace(api.workspace_bytes(n, d, H, **kw), "cuda")
        ws.fill_(0xCD)
        api.forward(x, x, x, seed=sd, workspace=ws, **kw)
        _sync()
        planes = region(ws, layout, "PLANES", np.uint8)
        f32 = planes[:H * r * d * 4].view(np.float32).reshape(H, r, d)
        off16 = (H * r * d * 4 + 255) // 256 * 256
        b16 = planes[off16:off16 + H * 16 * d * 2].view(np.uint16).reshape(H, 16, d)
        ref = osl.hyperplanes(sd, H, r, d)
        assert np.array_equal(f32.view(np.uint32), ref.view(np.uint32)), sd
        assert np.array_equal(b16[:, :r].astype(np.uint32) << 16, ref.view(np.uint32)), sd
        assert not b16[:, r:].any()
        assert np.array_equal(api.hyperplanes(sd, H, r, d), ref)


def test_first_call_of_a_fresh_seed_captured_in_a_graph():
    """The very first call with a new seed (and a new shape), rotary forward
    and backward, is captured in a HIP graph: the library allocates nothing
    and copies nothing from the host, so the capture holds kernels only.
    Three replays, with eager work and synchronisations between them, each
    equal the eager call with the same seed byte for byte and the oracle
    within tolerance."""
    banner("first call of a fresh seed in a HIP graph")
    import torch
    from oracle import rope as orope
    api = _api()
    w, Q, K, V, _ = _inputs("chatglm2_causal_n32768_d128_h32_bf16", heads=2, n=3072, b=96,
                            m=80, recursion_base=384, rope=False)
    dO = wl.make_grad(w)
    seed = 0x5EED_F1E5
    kw = dict(causal=True, b=w.b, m=w.m, r=w.r, recursion_base=w.recursion_base, seed=seed)
    q, k, v, do = (to_dev(x, "bf16") for x in (Q, K, V, dO))
    tab = api.rope_device_table(w.n, w.d, 10000.0, q.device)
    ws_f = api.alloc_workspace(api.workspace_bytes(w.n, w.d, w.heads, causal=True, b=w.b, m=w.m,
                                                   r=w.r, recursion_base=w.recursion_base),
                               "cuda")
    ws_b = api.alloc_workspace(api.backward_workspace_bytes(
        w.n, w.d, w.heads, causal=True, b=w.b, m=w.m, r=w.r, recursion_base=w.recursion_base),
        "cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o, lse, qr, kr = api.forward_rope(q, k, v, return_lse=True, return_rotated=True,
                                          workspace=ws_f, cos_sin=tab, **kw)
        grads = api.backward_rope(qr, kr, v, o, lse, do, workspace=ws_b, cos_sin=tab, **kw)
    outs = (o, lse, qr, kr) + tuple(grads)
    replays = []
    for rep in range(3):
        for t in outs:
            t.zero_()
        (q.float() * 2).sum().item()          # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        replays.append([t.clone() for t in outs])
    eo, else_, eqr, ekr = api.forward_rope(q, k, v, return_lse=True, return_rotated=True,
                                           cos_sin=tab, **kw)
    egrads = api.backward_rope(eqr, ekr, v, eo, else_, do, cos_sin=tab, **kw)
    torch.cuda.synchronize()
    for rep, got in enumerate(replays):
        for a_, b_ in zip(got, (eo, else_, eqr, ekr) + tuple(egrads)):
            assert torch.equal(a_, b_), rep
    ang = orope.angle_table(w.n, w.d, 10000.0)
    Qo = np.stack([orope.rope(Q[h], dtype="bf16", table=ang) for h in range(w.heads)])
    Ko = np.stack([orope.rope(K[h], dtype="bf16", table=ang) for h in range(w.heads)])
    Oref, Lref = oha.hyperattention(Qo, Ko, V, **kw)
    assert max_rel(to_np(replays[0][0]), Oref) <= TOL["bf16"]
    assert np.abs(to_np(replays[0][1]) - Lref).max() <= TOL["bf16"]


@pytest.mark.parametrize("causal", [True, False])
def test_debug_artifacts_match_oracle_and_forward(causal):
    """hyperattn_debug_artifacts copies the front end's results to the host:
    bit-exact against the oracle's artefacts and against the regions a
    forward call leaves in its workspace."""
    banner(f"debug artifacts causal={causal}")
    api = _api()
    if causal:
        w, Q, K, V, _ = _inputs("chatglm2_causal_n32768_d128_h32_bf16", heads=2, n=4096, b=128,
                                m=100, recursion_base=512)
    else:
        w, Q, K, V, _ = _inputs("single_head_noncausal_n1024_d64_fp32", heads=3, n=2048, b=128,
                                m=96)
    q, k, v = (to_dev(x, w.dtype) for x in (Q, K, V))
    arts = api.debug_artifacts(q, k, v, causal=w.causal, b=w.b, m=w.m, r=w.r,
                               recursion_base=w.recursion_base, seed=w.method_seed)
    art = {}
    oha.hyperattention(Q, K, V, causal=w.causal, b=w.b, m=w.m, r=w.r,
                       recursion_base=w.recursion_base, seed=w.method_seed,
                       rows=np.zeros(0, dtype=np.int64), artifacts=art)
    check_artifacts(w, None, None, art, list(range(w.heads)),
                    get=lambda name, dtype: arts[name].view(dtype))
    _, _, ws, layout = _run_forward(w, Q, K, V)
    for name in arts:
        assert np.array_equal(arts[name].view(np.uint8), region(ws, layout, name, np.uint8)), name


def test_rope_table_serves_shorter_and_grows():
    """One rotary table per (d, base) on the device, indexed by position: a
    longer call grows it, a shorter one reads its first rows. The rotated rows
    stay bit-exact throughout."""
    banner("rope table growth")
    from oracle import rope as orope
    api = _api()
    for n in (512, 2048, 512, 1024):
        w, Q, K, V, _ = _inputs("chatglm2_causal_n32768_d128_h32_bf16", heads=1, n=n, b=128,
                                m=64, recursion_base=256, rope=False)
        q, k, v = (to_dev(x, "bf16") for x in (Q, K, V))
        _, qr, kr = api.forward_rope(q, k, v, causal=True, b=w.b, m=w.m,
                                     recursion_base=w.recursion_base, rope_base=5000.0,
                                     return_rotated=True)
        _sync()
        tab = orope.angle_table(n, w.d, 5000.0)
        assert np.array_equal(to_np(qr)[0], orope.rope(Q[0], dtype="bf16", table=tab)), n
        assert np.array_equal(to_np(kr)[0], orope.rope(K[0], dtype="bf16", table=tab)), n


def test_persistent_grids_follow_each_kernels_occupancy():
    """Persistent launches size their grid from the occupancy of the kernel
    they launch: bf16 d = 64 attention kernels fit two work-groups per CU,
    d = 128 ones one, whichever runs first in the process."""
    banner("persistent grid per kernel")
    import torch
    api = _api()
    groups = {}
    for d in (128, 64, 128):
        x = torch.randn((4, 65536, d), device="cuda", dtype=torch.bfloat16)
        with api.KernelTimer() as t:
            api.forward(x, x, x, causal=False, b=256, m=256, seed=1)
            api.forward(x, x, x, causal=True, b=256, m=256, recursion_base=4096, seed=1)
            _sync()
        got = (t.groups["bucket_attention"] // 2, t.groups["exact_base_merge"])
        assert d not in groups or groups[d] == got, (d, groups[d], got)
        groups[d] = got
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"resident groups: d=128 {groups[128]}, d=64 {groups[64]} on {cus} CUs", flush=True)
    assert groups[64][0] == 2 * groups[128][0] == 2 * cus
    assert groups[64][1] == 2 * groups[128][1] == 2 * cus
