"""The allocation-free forward (hyperattn_forward_noalloc, whose workspace is
the library's static per-GPU scratch) through the C ABI, against
hyperattn_forward with a caller workspace: two calls in a row, the second
with a smaller input, each byte-equal to the workspace entry point's output;
sizes beyond the scratch are refused before anything is enqueued."""

import ctypes

import numpy as np
import pytest

from approximate_softmax_attention_amd import workloads as wl
from tests.gpu_util import banner, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # the long-context non-causal workload at full size (40 MiB of workspace)
    ("longctx_noncausal_n131072_d64_h8_bf16", {}),
    # then a smaller causal input with recursion, merge and another d
    ("chatglm2_causal_n32768_d128_h32_bf16",
     dict(heads=2, n=4096, b=128, m=100, recursion_base=512)),
]


def _noalloc(lib, q, k, v, o, lse, w):
    import torch
    H, n, d = q.shape
    return lib.hyperattn_forward_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
        ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()),
        ctypes.c_void_p(lse.data_ptr()), n, d, H, int(w.causal), w.b, w.m, w.recursion_base,
        w.r, w.method_seed, 1, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_forward_equals_the_workspace_forward():
    import torch
    from approximate_softmax_attention_amd import _lib, api
    lib = _lib.lib()
    scratch = lib.hyperattn_noalloc_scratch_bytes()
    assert scratch == 64 << 20
    for name, changes in CASES:
        w = wl.scaled(wl.WORKLOADS[name], **changes) if changes else wl.WORKLOADS[name]
        banner(f"no-alloc forward {w.name} heads={w.heads} n={w.n} d={w.d}")
        need = api.workspace_bytes(w.n, w.d, w.heads, causal=w.causal, b=w.b, m=w.m, r=w.r,
                                   recursion_base=w.recursion_base)
        assert 0 < need <= scratch
        Q, K, V, _ = wl.make_inputs_parallel(w)
        q, k, v = (to_dev(x, "bf16") for x in (Q, K, V))
        o = torch.full_like(q, float("nan"))
        lse = torch.full((w.heads, w.n), float("nan"), device="cuda")
        assert _noalloc(lib, q, k, v, o, lse, w) == 0, _lib.last_error()
        ref, ref_lse = api.forward(q, k, v, causal=w.causal, b=w.b, m=w.m, r=w.r,
                                   recursion_base=w.recursion_base, seed=w.method_seed,
                                   return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o, ref) and torch.equal(lse, ref_lse), w.name


def test_noalloc_refuses_sizes_beyond_the_scratch():
    import torch
    from approximate_softmax_attention_amd import _lib
    lib = _lib.lib()
    w = wl.scaled(wl.WORKLOADS["chatglm2_causal_n32768_d128_h32_bf16"], heads=8)
    q = torch.zeros((8, w.n, w.d), device="cuda", dtype=torch.bfloat16)
    o = torch.zeros_like(q)
    lse = torch.zeros((8, w.n), device="cuda")
    rc = _noalloc(lib, q, q, q, o, lse, w)
    assert rc == -4 and "static scratch" in _lib.last_error()
    torch.cuda.synchronize()
    assert not o.any()
