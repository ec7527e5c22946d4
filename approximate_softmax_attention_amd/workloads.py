"""Seeded synthetic workloads shared by the tests and the benchmark.

This module only makes inputs: it holds none of the attention method's
arithmetic and imports neither the HIP binding nor the CPU oracle.

Recipe (numpy only, deterministic):

* Every (data seed, tensor, head) triple has its own PCG64 stream that draws
  float64 standard normals of shape [n, d]. Tensor ids: Q = 0, K = 1, V = 2,
  planting = 3, the output gradient dO of the backward pass = 4.
* Optional planting of heavy entries (the 8-head, n = 8192 workload): queries
  are visited in index order; each picks 4 distinct keys uniformly at random
  and overwrites them with 3 sqrt(d) q / ||q|| plus N(0, 0.1^2) noise per
  coordinate. A later overwrite wins; the surviving (query, key) pairs are
  returned as ground truth.
* Optional rotary position embedding on Q and K (the causal long-context
  workloads): coordinate pairs (t, t + d/2) at position p are rotated by the
  angle p * 10000^(-2t/d).
* Values are then rounded to fp32 and, for bf16 workloads, to bf16 by
  round-to-nearest-even on the fp32 bit pattern. Both sides of every parity
  check read these same bytes.
* Very long single heads (make_inputs_large, for the tests at the largest
  sizes the library takes) draw the same distribution in row chunks of
  2^18, chunk c of (data seed, tensor, head) from its own PCG64 stream
  [data seed, tensor, head, c + 1], on a thread pool.
"""

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    n: int
    d: int
    dtype: str            # "fp32" or "bf16"
    causal: bool
    b: int
    m: int
    r: int = 8
    recursion_base: int = 4096
    rope: bool = False
    planted: int = 0      # heavy keys planted per query (0: none)
    data_seed: int = 0
    method_seed: int = 0
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "single_head_noncausal_n1024_d64_fp32": Workload(
        "single_head_noncausal_n1024_d64_fp32", 1, 1024, 64, "fp32", False,
        128, 128, data_seed=1, method_seed=1001,
        notes="iid N(0,1); scores scaled by 1/sqrt(d)"),
    "planted_noncausal_n8192_d64_h8_bf16": Workload(
        "planted_noncausal_n8192_d64_h8_bf16", 8, 8192, 64, "bf16", False,
        256, 256, planted=4, data_seed=2, method_seed=1002,
        notes="iid N(0,1) with 4 planted heavy keys per query"),
    "chatglm2_causal_n32768_d128_h32_bf16": Workload(
        "chatglm2_causal_n32768_d128_h32_bf16", 32, 32768, 128, "bf16", True,
        256, 256, rope=True, data_seed=3, method_seed=1003,
        notes="ChatGLM2-6B-shaped layer; RoPE on Q, K"),
    "longctx_causal_n131072_d128_h32_bf16": Workload(
        "longctx_causal_n131072_d128_h32_bf16", 32, 131072, 128, "bf16", True,
        256, 256, rope=True, data_seed=4, method_seed=1004,
        notes="long-context causal layer; RoPE on Q, K"),
    "longctx_noncausal_n131072_d64_h8_bf16": Workload(
        "longctx_noncausal_n131072_d64_h8_bf16", 8, 131072, 64, "bf16", False,
        256, 256, data_seed=5, method_seed=1005,
        notes="long-context non-causal layer"),
}

HEADLINE = "longctx_causal_n131072_d128_h32_bf16"

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_PLANT, TENSOR_DO = 0, 1, 2, 3, 4


def normals(data_seed, tensor, head, n, d):
    g = np.random.Generator(np.random.PCG64([data_seed, tensor, head]))
    return g.standard_normal((n, d))


def rope(X):
    """Rotary embedding with base 10000 on rows at positions 0 .. n-1 (fp64)."""
    n, d = X.shape
    half = d // 2
    theta = 10000.0 ** (-2.0 * np.arange(half) / d)
    ang = np.arange(n, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = X[:, :half], X[:, half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=1)


def plant(Q, K, data_seed, head, per_query):
    """Overwrite keys with scaled copies of queries; returns surviving pairs."""
    n, d = Q.shape
    g = np.random.Generator(np.random.PCG64([data_seed, TENSOR_PLANT, head]))
    owner = np.full(n, -1, dtype=np.int64)
    for i in range(n):
        js = g.choice(n, size=per_query, replace=False)
        qn = Q[i] / np.linalg.norm(Q[i])
        for j in js:
            K[j] = 3.0 * np.sqrt(d) * qn + 0.1 * g.standard_normal(d)
            owner[j] = i
    keys = np.nonzero(owner >= 0)[0]
    return np.stack([owner[keys], keys], axis=1)


def f32_to_bf16_bits(x32):
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def make_head(w, head):
    """One head's (Q, K, V) as fp32 arrays holding exactly the stored values,
    plus the planted pairs (or None)."""
    Q = normals(w.data_seed, TENSOR_Q, head, w.n, w.d)
    K = normals(w.data_seed, TENSOR_K, head, w.n, w.d)
    V = normals(w.data_seed, TENSOR_V, head, w.n, w.d)
    pairs = plant(Q, K, w.data_seed, head, w.planted) if w.planted else None
    if w.rope:
        Q, K = rope(Q), rope(K)
    out = []
    for X in (Q, K, V):
        x32 = X.astype(np.float32)
        if w.dtype == "bf16":
            x32 = bf16_bits_to_f32(f32_to_bf16_bits(x32))
        out.append(x32)
    return out[0], out[1], out[2], pairs


def make_inputs(w, heads=None):
    """All heads (or the listed ones): fp32 arrays [H, n, d] and planted pairs."""
    hs = range(w.heads) if heads is None else heads
    Qs, Ks, Vs, P = [], [], [], []
    for h in hs:
        q, k, v, p = make_head(w, h)
        Qs.append(q), Ks.append(k), Vs.append(v), P.append(p)
    return np.stack(Qs), np.stack(Ks), np.stack(Vs), P


def make_grad(w, heads=None):
    """Output gradients dO [H, n, d] for the backward pass: standard normals,
    rounded like the inputs."""
    hs = range(w.heads) if heads is None else heads
    out = []
    for h in hs:
        x32 = normals(w.data_seed, TENSOR_DO, h, w.n, w.d).astype(np.float32)
        if w.dtype == "bf16":
            x32 = bf16_bits_to_f32(f32_to_bf16_bits(x32))
        out.append(x32)
    return np.stack(out)


def make_inputs_large(w, chunk=1 << 18, workers=None):
    """(Q, K, V) as fp32 arrays [heads, n, d] for very long heads: iid N(0, 1)
    in row chunks, each from its own stream, generated in parallel (no
    planting or RoPE), rounded like make_head's values."""
    import concurrent.futures as cf
    import os
    if w.planted or w.rope:
        raise ValueError("make_inputs_large draws plain iid inputs only")
    workers = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    out = [np.empty((w.heads, w.n, w.d), dtype=np.float32) for _ in range(3)]
    jobs = [(t, h, c) for t in range(3) for h in range(w.heads)
            for c in range((w.n + chunk - 1) // chunk)]

    def fill(job):
        t, h, c = job
        lo, hi = c * chunk, min(w.n, (c + 1) * chunk)
        g = np.random.Generator(np.random.PCG64([w.data_seed, t, h, c + 1]))
        x32 = g.standard_normal((hi - lo, w.d)).astype(np.float32)
        if w.dtype == "bf16":
            x32 = bf16_bits_to_f32(f32_to_bf16_bits(x32))
        out[t][h, lo:hi] = x32

    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, jobs))
    return out[0], out[1], out[2]


def make_inputs_parallel(w, heads=None, workers=None):
    """make_inputs with heads generated on a thread pool (numpy releases the GIL)."""
    import concurrent.futures as cf
    import os
    hs = list(range(w.heads)) if heads is None else list(heads)
    workers = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(lambda h: make_head(w, h), hs))
    return (np.stack([r[0] for r in res]), np.stack([r[1] for r in res]),
            np.stack([r[2] for r in res]), [r[3] for r in res])


def scaled(w, **changes):
    """A copy of a workload with some fields replaced (smaller test shapes)."""
    d = dict(w.__dict__)
    d.update(changes)
    return Workload(**d)
