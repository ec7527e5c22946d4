"""Rotary position embedding before hashing (test infrastructure only).

The workloads of the long-context layers apply RoPE to Q and K, and the hash
then sees the rotated rows (HA page, "Algorithm": sortLSH hashes the rows the
attention uses). Reading taken, the usual rotary form:

* pairs (t, t + d/2) for t < d/2, frequency theta_t = base^(-2t/d), row i at
  position i;
* x'_t       = x_t cos(i theta_t) - x_{t+d/2} sin(i theta_t)
  x'_{t+d/2} = x_t sin(i theta_t) + x_{t+d/2} cos(i theta_t)
  in fp32, every product and the sum rounded once (no fused multiply-add),
  with cos and sin rounded to fp32;
* pow, cos and sin are the C library's (Python's math module): theta_t, the
  angle i * theta_t, cos and sin are fp64 values;
* for bf16 rows the result is rounded to the nearest bf16 (ties to even).
The fp32 rotation errs by about 1e-7 relative, far inside a bf16 step.

The gradient through the embedding (rope_adjoint) is the transpose of the
rotation: each pair's rotation is orthogonal, so the transpose turns by
-i theta_t. The bf16 rounding of the rotated rows is piecewise constant and
carries no gradient (the reading the backward pass takes for the sketch).
"""

import math

import numpy as np


def angle_table(n, d, base):
    """cos and sin of i * theta_t, [n, d/2] each, fp64 from the C library."""
    half = d // 2
    theta = [math.pow(base, -2.0 * t / d) for t in range(half)]
    c = np.empty((n, half))
    s = np.empty((n, half))
    for i in range(n):
        for t in range(half):
            a = float(i) * theta[t]
            c[i, t] = math.cos(a)
            s[i, t] = math.sin(a)
    return c, s


def round_bf16_array(x32):
    """Nearest bfloat16 values (ties to even) of an fp32 array, as fp32."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return (u & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def rope(X, base=10000.0, dtype="bf16", table=None):
    """Rotated copy of X [n, d] (fp32 array holding the input values)."""
    n, d = X.shape
    half = d // 2
    c, s = table if table is not None else angle_table(n, d, base)
    c = np.asarray(c, dtype=np.float32)
    s = np.asarray(s, dtype=np.float32)
    x1 = np.asarray(X[:, :half], dtype=np.float32)
    x2 = np.asarray(X[:, half:], dtype=np.float32)
    a = x1 * c                       # fp32 products and sums, each rounded once
    b = x2 * s
    e = x1 * s
    f = x2 * c
    out = np.concatenate([a - b, e + f], axis=1).astype(np.float32)
    return round_bf16_array(out) if dtype == "bf16" else out


def rope_adjoint(G, base=10000.0, dtype="fp64", table=None):
    """Gradient of the rows before rotation, from G [n, d], the gradient of
    the rotated rows: the transpose of each pair's rotation,
      g_t       =  g'_t cos(i theta_t) + g'_{t+d/2} sin(i theta_t)
      g_{t+d/2} = -g'_t sin(i theta_t) + g'_{t+d/2} cos(i theta_t).
    dtype "fp64": exact arithmetic on the fp64 table; "fp32" / "bf16": fp32
    cos, sin, products and sums each rounded once, then (bf16) rounded to
    the nearest bf16."""
    n, d = G.shape
    half = d // 2
    c, s = table if table is not None else angle_table(n, d, base)
    ft = np.float64 if dtype == "fp64" else np.float32
    c = np.asarray(c, dtype=ft)
    s = np.asarray(s, dtype=ft)
    g1 = np.asarray(G[:, :half], dtype=ft)
    g2 = np.asarray(G[:, half:], dtype=ft)
    out = np.concatenate([g1 * c + g2 * s, g2 * c - g1 * s], axis=1).astype(ft)
    return round_bf16_array(out) if dtype == "bf16" else out
