"""GPU parity of the backward pass: the library's gradients through its C ABI
against the oracle's (oracle.backward) on the shared seeded inputs.

Tolerance: the gradients are bf16 outputs of bf16 inputs with fp32
accumulation, compared as max |g - g_ref| / max |g_ref| per head against the
bf16 bound of gpu_util.TOL. The library differentiates its own forward
output (bf16 O, fp32 lse), the oracle its fp64 one.
"""

import numpy as np
import pytest

from approximate_softmax_attention_amd import workloads as wl
from oracle import backward as obw
from tests.gpu_util import TOL, banner, max_rel, to_dev, to_np

pytestmark = pytest.mark.gpu


def _api():
    from approximate_softmax_attention_amd import api
    return api


def _sync():
    import torch
    torch.cuda.synchronize()


def _errs(grads, refs):
    return [max_rel(to_np(g), r) for g, r in zip(grads, refs)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [77, 300])
def test_exact_backward(d, causal, n):
    banner(f"exact backward d={d} causal={causal} n={n}")
    w = wl.scaled(wl.WORKLOADS["single_head_noncausal_n1024_d64_fp32"], heads=2, n=n, d=d,
                  dtype="bf16")
    Q, K, V, _ = wl.make_inputs(w)
    dO = wl.make_grad(w)
    api = _api()
    q, k, v, do = (to_dev(x, "bf16") for x in (Q, K, V, dO))
    o, lse = api.exact(q, k, v, causal=causal, return_lse=True)
    grads = api.exact_backward(q, k, v, o, lse, do, causal=causal)
    _sync()
    refs = [np.stack([obw.exact_attention_backward(Q[h], K[h], V[h], dO[h], causal=causal)[i]
                      for h in range(2)]) for i in range(3)]
    errs = _errs(grads, refs)
    print(f"  dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e}", flush=True)
    assert max(errs) <= TOL["bf16"], errs


BACKWARD_CASES = {
    # non-causal, samples smaller than n, d = 64
    "noncausal_d64": ("planted_noncausal_n8192_d64_h8_bf16",
                      dict(heads=2, n=1024, b=128, m=128, planted=0)),
    # causal, two levels and a base case, d = 128
    "causal_d128": ("chatglm2_causal_n32768_d128_h32_bf16",
                    dict(heads=2, n=2048, b=128, m=128, recursion_base=512, rope=False)),
    # causal, three levels, the last one with exhaustive samples (m >= n_k)
    "causal_exhaustive": ("chatglm2_causal_n32768_d128_h32_bf16",
                          dict(heads=1, n=1024, d=64, b=64, m=200, recursion_base=128,
                               rope=False)),
    # the local block mask (r = 0)
    "local_mask": ("planted_noncausal_n8192_d64_h8_bf16",
                   dict(heads=2, n=1024, b=128, m=64, r=0, planted=0)),
    # buckets of 512 rows: two query / key chunks per bucket
    "wide_bucket": ("longctx_noncausal_n131072_d64_h8_bf16",
                    dict(heads=1, n=2048, d=128, b=512, m=256)),
    # 16384 rows: the sample slots' gradient takes two query chunks
    "two_query_chunks": ("longctx_noncausal_n131072_d64_h8_bf16",
                         dict(heads=1, n=16384, b=256, m=256)),
    # causal with n <= recursion_base: the whole problem is one base block
    "causal_base_only": ("chatglm2_causal_n32768_d128_h32_bf16",
                         dict(heads=2, n=384, b=128, m=128, recursion_base=512, rope=False)),
    # one bucket holds every key: every sample lies inside the query's bucket
    "bucket_covers_n": ("planted_noncausal_n8192_d64_h8_bf16",
                        dict(heads=1, n=512, b=512, m=64, planted=0)),
    # d = 128 with slot lists that are not whole 128-slot groups (m = 200) and
    # a last level with exhaustive samples
    "causal_exhaustive_d128": ("chatglm2_causal_n32768_d128_h32_bf16",
                               dict(heads=1, n=1024, b=64, m=200, recursion_base=128,
                                    rope=False)),
    # the sizes of the forward's bf16 slot-window refill (b + 2m > 1024)
    "slot_refill_d128": ("chatglm2_causal_n32768_d128_h32_bf16",
                         dict(heads=1, n=8192, b=512, m=300, recursion_base=1024, rope=False)),
}


def _run_case(name, zero_v_half=False):
    base, changes = BACKWARD_CASES[name]
    w = wl.scaled(wl.WORKLOADS[base], **changes)
    Q, K, V, _ = wl.make_inputs(w)
    if zero_v_half:
        V[:, : w.n // 2] = 0.0
    dO = wl.make_grad(w)
    api = _api()
    q, k, v, do = (to_dev(x, "bf16") for x in (Q, K, V, dO))
    kw = dict(causal=w.causal, b=w.b, m=w.m, r=w.r, recursion_base=w.recursion_base,
              seed=w.method_seed)
    o, lse = api.forward(q, k, v, return_lse=True, **kw)
    grads = api.backward(q, k, v, o, lse, do, **kw)
    _sync()
    refs = obw.hyperattention_backward(Q, K, V, dO, causal=w.causal, b=w.b, m=w.m, r=w.r,
                                       recursion_base=w.recursion_base, seed=w.method_seed)
    return w, (q, k, v, o, lse, do, kw), grads, refs


@pytest.mark.parametrize("name", list(BACKWARD_CASES))
def test_hyperattention_backward(name):
    banner(f"hyperattention backward {name}")
    _, _, grads, refs = _run_case(name)
    errs = _errs(grads, refs)
    print(f"  dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e}", flush=True)
    assert max(errs) <= TOL["bf16"], errs


@pytest.mark.parametrize("name", ["causal_exhaustive", "causal_exhaustive_d128"])
def test_backward_empty_vnorm_list(name):
    """V rows [0, n/2) all zero: the first level's node draws no V-norm
    sample, so its keys get no product gradient from samples."""
    banner(f"hyperattention backward with an empty V-norm list ({name})")
    _, _, grads, refs = _run_case(name, zero_v_half=True)
    errs = _errs(grads, refs)
    print(f"  dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e}", flush=True)
    assert max(errs) <= TOL["bf16"], errs


def test_backward_deterministic_and_autograd():
    """Two calls give the same bytes, and the autograd wrapper returns them."""
    banner("hyperattention backward determinism and autograd")
    import torch
    _, (q, k, v, o, lse, do, kw), grads, _ = _run_case("causal_d128")
    api = _api()
    again = api.backward(q, k, v, o, lse, do, **kw)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    out = api.HyperAttentionFunction.apply(qa, ka, va, kw["causal"], kw["b"], kw["m"], kw["r"],
                                           kw["recursion_base"], kw["seed"])
    out.backward(do)
    _sync()
    assert torch.equal(out.detach(), o)
    for g, h, t in zip(grads, again, (qa, ka, va)):
        assert torch.equal(g, h)
        assert torch.equal(g, t.grad)


def test_backward_batch_dimension_folds_into_heads():
    """[batch, heads, n, d] tensors give the gradients of the same call on
    [batch * heads, n, d]."""
    banner("hyperattention backward with a batch dimension")
    import torch
    (q, k, v, o, lse, do, kw) = _run_case("noncausal_d64")[1]
    api = _api()
    H, n, d = q.shape
    shape4 = (2, H // 2, n, d)
    g3 = api.backward(q, k, v, o, lse, do, **kw)
    g4 = api.backward(q.reshape(shape4), k.reshape(shape4), v.reshape(shape4),
                      o.reshape(shape4), lse.reshape(2, H // 2, n), do.reshape(shape4), **kw)
    _sync()
    for a, b in zip(g3, g4):
        assert b.shape == shape4
        assert torch.equal(a, b.reshape(a.shape))


@pytest.mark.parametrize("name", ["causal_d128", "local_mask"])
def test_backward_rope(name):
    """hyperattn_backward_rope: the gradients of the rows before their rotary
    embedding, against the oracle's backward on the oracle-rotated rows
    followed by the oracle's fp64 transposed rotation; the autograd wrapper
    returns the same bytes."""
    banner(f"hyperattention backward through RoPE ({name})")
    import torch
    from oracle import rope as orope
    base, changes = BACKWARD_CASES[name]
    w = wl.scaled(wl.WORKLOADS[base], **changes)
    Q, K, V, _ = wl.make_inputs(w)
    dO = wl.make_grad(w)
    api = _api()
    q, k, v, do = (to_dev(x, "bf16") for x in (Q, K, V, dO))
    kw = dict(causal=w.causal, b=w.b, m=w.m, r=w.r, recursion_base=w.recursion_base,
              seed=w.method_seed)
    o, lse, qr, kr = api.forward_rope(q, k, v, return_lse=True, return_rotated=True, **kw)
    grads = api.backward_rope(qr, kr, v, o, lse, do, **kw)
    plain = api.backward(qr, kr, v, o, lse, do, **kw)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    out = api.HyperAttentionRopeFunction.apply(qa, ka, va, kw["causal"], kw["b"], kw["m"],
                                               kw["r"], kw["recursion_base"], kw["seed"],
                                               10000.0)
    out.backward(do)
    _sync()
    assert torch.equal(plain[2], grads[2])         # dV does not see the rotation
    assert torch.equal(out.detach(), o)
    for g, t in zip(grads, (qa, ka, va)):
        assert torch.equal(g, t.grad)
    tab = orope.angle_table(w.n, w.d, 10000.0)
    Qo = np.stack([orope.rope(Q[h], dtype="bf16", table=tab) for h in range(w.heads)])
    Ko = np.stack([orope.rope(K[h], dtype="bf16", table=tab) for h in range(w.heads)])
    assert np.array_equal(to_np(qr), Qo) and np.array_equal(to_np(kr), Ko)
    dq, dk, dv = obw.hyperattention_backward(Qo, Ko, V, dO, causal=w.causal, b=w.b, m=w.m,
                                             r=w.r, recursion_base=w.recursion_base,
                                             seed=w.method_seed)
    refs = [np.stack([orope.rope_adjoint(g[h], table=tab) for h in range(w.heads)])
            for g in (dq, dk)] + [dv]
    errs = _errs(grads, refs)
    print(f"  dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e}", flush=True)
    assert max(errs) <= TOL["bf16"], errs


def test_forward_and_backward_replay_in_a_hip_graph():
    """A forward + backward call enqueues only kernels on the caller's stream
    (the hyperplanes are drawn on the device), so it can be captured in a HIP
    graph. Three replays, with eager work and synchronisations between them,
    each equal the eager result byte for byte."""
    banner("forward + backward in a HIP graph")
    import torch
    base, changes = BACKWARD_CASES["causal_d128"]
    w = wl.scaled(wl.WORKLOADS[base], **changes)
    Q, K, V, _ = wl.make_inputs(w)
    dO = wl.make_grad(w)
    api = _api()
    q, k, v, do = (to_dev(x, "bf16") for x in (Q, K, V, dO))
    kw = dict(causal=w.causal, b=w.b, m=w.m, r=w.r, recursion_base=w.recursion_base,
              seed=w.method_seed)
    ws_f = api.alloc_workspace(api.workspace_bytes(w.n, w.d, w.heads, causal=w.causal, b=w.b,
                                                   m=w.m, r=w.r,
                                                   recursion_base=w.recursion_base), "cuda")
    ws_b = api.alloc_workspace(api.backward_workspace_bytes(
        w.n, w.d, w.heads, causal=w.causal, b=w.b, m=w.m, r=w.r,
        recursion_base=w.recursion_base), "cuda")
    o = torch.empty_like(q)
    lse = torch.empty((w.heads, w.n), dtype=torch.float32, device="cuda")

    def step():
        api.forward(q, k, v, out=o, lse_out=lse, workspace=ws_f, **kw)
        return api.backward(q, k, v, o, lse, do, workspace=ws_b, **kw)

    eager = [t.clone() for t in step()]
    eager_o = o.clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        grads = step()
    for rep in range(3):
        o.zero_()
        for t in grads:
            t.zero_()
        (q.float() * 2).sum().item()          # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager_o), rep
        for a, b in zip(grads, eager):
            assert torch.equal(a, b), rep
