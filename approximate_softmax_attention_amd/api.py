"""PyTorch-facing binding of libhyperattn.so.

Argument marshalling only: tensors are checked, outputs and workspaces are
allocated with torch on the tensors' device, and the library is called on
torch's current HIP stream. Every step of the computation runs in the
library's HIP kernels; there is no other code path.

Tensors are [heads, n, d] (or [batch, heads, n, d], folded into heads),
contiguous, on a ROCm device, dtype torch.bfloat16 or torch.float32 (the
backward pass takes bfloat16).

Entry points: forward, forward_rope, backward, backward_rope, exact, exact_backward,
rowsum_estimate, sortlsh_hash, hyperplanes, gaussians, rope_table,
rope_device_table, debug_artifacts, workspace_bytes, backward_workspace_bytes,
workspace_layout; HyperAttentionFunction and
HyperAttentionRopeFunction wrap forward and backward for torch.autograd; KernelTimer collects the library's
per-kernel hipEvent timings.
"""

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import HA_BF16, HA_F32, check, lib


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return HA_BF16
    if t.dtype == torch.float32:
        return HA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _fold(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() == 4:
        return t.reshape(t.shape[0] * t.shape[1], t.shape[2], t.shape[3])
    if t.dim() != 3:
        raise ValueError(f"{name} must be [heads, n, d] or [batch, heads, n, d]")
    return t


def _qkv(q, k, v=None):
    shape = q.shape
    q, k = _fold(q, "q"), _fold(k, "k")
    if v is not None:
        v = _fold(v, "v")
    for t in (k,) + ((v,) if v is not None else ()):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must have the same shape, dtype and device")
    return shape, q, k, v


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check_buffer(t, name, like, numel, dtype):
    """A caller-supplied output: contiguous, on `like`'s device, of `dtype`
    and `numel` elements (the library writes exactly that many)."""
    if t is None:
        return
    if t.device != like.device or t.dtype != dtype or not t.is_contiguous() or \
            t.numel() != numel:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of {numel} elements on "
                         f"{like.device}")


def _workspace(ws, nbytes, like):
    """The caller's workspace (a contiguous uint8 tensor on `like`'s device,
    its size checked by the library) or a new one of nbytes."""
    if ws is None:
        return alloc_workspace(nbytes, like.device)
    if ws.device != like.device or ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {like.device}")
    return ws


def _call(like, fn, *args, after=()):
    """Calls a library entry point with `like`'s device current (the library
    launches on the current device) on torch's current stream there; `after`
    are arguments that follow the stream."""
    with torch.cuda.device(like.device):
        check(fn(*args, _stream(like.device), *after))


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def workspace_bytes(n, d, heads, *, causal, b, m, r=8, recursion_base=4096, dtype=HA_BF16):
    nb = lib().hyperattn_workspace_bytes(n, d, heads, int(causal), b, m, recursion_base, r, dtype)
    if nb == 0 and _lib.last_error():
        raise _lib.HyperAttnError(-2, _lib.last_error())
    return nb


def alloc_workspace(nbytes, device):
    # torch's caching allocator returns blocks aligned to at least 512 bytes
    ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    assert ws.data_ptr() % 256 == 0
    return ws


def forward(q, k, v, *, causal, b=256, m=256, r=8, recursion_base=4096, seed=0,
            return_lse=False, workspace=None, out=None, lse_out=None):
    """HyperAttention forward; returns O (and lse if asked).

    r: hyperplanes per head for sortLSH (1..8), or 0 for the local block mask
    (bucket k = query and key rows [k b, (k+1) b) of each sub-problem).
    """
    shape, q, k, v = _qkv(q, k, v)
    H, n, d = q.shape
    dt = _dtype_code(q)
    _check_buffer(out, "out", q, q.numel(), q.dtype)
    _check_buffer(lse_out, "lse_out", q, H * n, torch.float32)
    o = out if out is not None else torch.empty_like(q)
    lse = lse_out
    if return_lse and lse is None:
        lse = torch.empty((H, n), dtype=torch.float32, device=q.device)
    nb = workspace_bytes(n, d, H, causal=causal, b=b, m=m, r=r,
                         recursion_base=recursion_base, dtype=dt)
    ws = _workspace(workspace, nb, q)
    _call(q, lib().hyperattn_forward, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), n, d, H,
          int(causal), b, m, recursion_base, r, seed, dt, _ptr(ws), ws.numel())
    o = o.reshape(shape)
    if return_lse:
        return o, lse.reshape(shape[:-1])
    return o


# Device copies of rope_table, one per (device, d, rope_base), indexed by
# position: a longer call replaces the table by one at least twice as long, a
# shorter call reads its first rows. torch owns the memory.
_ROPE_TABLES = {}


def rope_device_table(n, d, rope_base, device):
    """The cos/sin table of at least n positions on `device` (fp32 tensor
    [rows, d/2, 2]) for forward_rope and backward_rope."""
    key = (torch.device(device), int(d), float(rope_base))
    t = _ROPE_TABLES.get(key)
    if t is None or t.shape[0] < n:
        rows = max(int(n), 2 * t.shape[0] if t is not None else 0, 1)
        rows = min(rows, max(int(n), (1 << 31) - 1))
        t = torch.from_numpy(rope_table(rows, d, rope_base)).to(key[0])
        _ROPE_TABLES[key] = t
    return t


def _check_table(cos_sin, n, d, like):
    if cos_sin.device != like.device or cos_sin.dtype != torch.float32 or \
            not cos_sin.is_contiguous() or cos_sin.dim() != 3 or \
            tuple(cos_sin.shape[1:]) != (d // 2, 2) or cos_sin.shape[0] < n:
        raise ValueError(f"cos_sin must be a contiguous fp32 [>= {n}, {d // 2}, 2] tensor on "
                         f"{like.device}")
    return cos_sin


def forward_noalloc(q, k, v, *, causal, b=256, m=256, r=8, recursion_base=4096, seed=0,
                    out, lse_out=None):
    """hyperattn_forward_noalloc: the forward pass in the library's static
    per-GPU scratch, with caller-supplied outputs (nothing is allocated)."""
    shape, q, k, v = _qkv(q, k, v)
    H, n, d = q.shape
    _check_buffer(out, "out", q, q.numel(), q.dtype)
    _check_buffer(lse_out, "lse_out", q, H * n, torch.float32)
    _call(q, lib().hyperattn_forward_noalloc, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
          _ptr(lse_out), n, d, H, int(causal), b, m, recursion_base, r, seed, _dtype_code(q))
    return out.reshape(shape)


def forward_rope(q, k, v, *, causal, rope_base=10000.0, b=256, m=256, r=8,
                 recursion_base=4096, seed=0, return_lse=False, return_rotated=False,
                 workspace=None, cos_sin=None):
    """HyperAttention forward on Q and K before their rotary embedding, which
    the library applies on the device in the pass that hashes them; returns O
    (then lse, then the rotated Q and K, as asked). cos_sin: the device table
    (rope_device_table(n, d, rope_base, device) unless given)."""
    shape, q, k, v = _qkv(q, k, v)
    H, n, d = q.shape
    dt = _dtype_code(q)
    tab = _check_table(cos_sin if cos_sin is not None else
                       rope_device_table(n, d, rope_base, q.device), n, d, q)
    o = torch.empty_like(q)
    qr, kr = torch.empty_like(q), torch.empty_like(k)
    lse = torch.empty((H, n), dtype=torch.float32, device=q.device) if return_lse else None
    nb = workspace_bytes(n, d, H, causal=causal, b=b, m=m, r=r,
                         recursion_base=recursion_base, dtype=dt)
    ws = _workspace(workspace, nb, q)
    _call(q, lib().hyperattn_forward_rope, _ptr(q), _ptr(k), _ptr(v), _ptr(tab), tab.shape[0],
          _ptr(qr), _ptr(kr), _ptr(o), _ptr(lse), n, d, H, int(causal), b, m, recursion_base, r,
          seed, dt, _ptr(ws), ws.numel())
    out = [o.reshape(shape)]
    if return_lse:
        out.append(lse.reshape(shape[:-1]))
    if return_rotated:
        out += [qr.reshape(shape), kr.reshape(shape)]
    return out[0] if len(out) == 1 else tuple(out)


def rope_table(n, d, rope_base=10000.0):
    """The cos/sin table of forward_rope, [n, d/2, 2] fp32 (host computation)."""
    T = np.empty((n, d // 2, 2), dtype=np.float32)
    check(lib().rope_table(n, d, float(rope_base),
                           T.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
    return T


def exact(q, k, v, *, causal=False, return_lse=False, out=None, lse_out=None):
    """Exact softmax attention (the library's own kernel)."""
    shape, q, k, v = _qkv(q, k, v)
    H, n, d = q.shape
    _check_buffer(out, "out", q, q.numel(), q.dtype)
    _check_buffer(lse_out, "lse_out", q, H * n, torch.float32)
    o = out if out is not None else torch.empty_like(q)
    lse = lse_out
    if return_lse and lse is None:
        lse = torch.empty((H, n), dtype=torch.float32, device=q.device)
    _call(q, lib().exact_attention_forward, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), n, d,
          H, int(causal), _dtype_code(q))
    o = o.reshape(shape)
    if return_lse:
        return o, lse.reshape(shape[:-1])
    return o


def _grad_inputs(q, k, v, o, lse, do):
    shape, q, k, v = _qkv(q, k, v)
    o, do = _fold(o, "o"), _fold(do, "do")
    for t, name in ((o, "o"), (do, "do")):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must have the shape, dtype and device of q")
    H, n, _ = q.shape
    if lse.device != q.device or not lse.is_contiguous() or lse.dtype != torch.float32 or \
            lse.numel() != H * n:
        raise ValueError("lse must be the forward pass's contiguous fp32 [heads, n] output")
    return shape, q, k, v, o, lse, do


def backward_workspace_bytes(n, d, heads, *, causal, b, m, r=8, recursion_base=4096,
                             dtype=HA_BF16):
    nb = lib().hyperattn_backward_workspace_bytes(n, d, heads, int(causal), b, m,
                                                  recursion_base, r, dtype)
    if nb == 0 and _lib.last_error():
        raise _lib.HyperAttnError(-3, _lib.last_error())
    return nb


def backward(q, k, v, o, lse, do, *, causal, b=256, m=256, r=8, recursion_base=4096, seed=0,
             workspace=None):
    """Gradients (dq, dk, dv) of sum(do * o) for o, lse = forward(q, k, v, ...,
    return_lse=True) with the same arguments (bf16 tensors)."""
    shape, q, k, v, o, lse, do = _grad_inputs(q, k, v, o, lse, do)
    H, n, d = q.shape
    dt = _dtype_code(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nb = backward_workspace_bytes(n, d, H, causal=causal, b=b, m=m, r=r,
                                  recursion_base=recursion_base, dtype=dt)
    ws = _workspace(workspace, nb, q)
    _call(q, lib().hyperattn_backward, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
          _ptr(dq), _ptr(dk), _ptr(dv), n, d, H, int(causal), b, m, recursion_base, r, seed, dt,
          _ptr(ws), ws.numel())
    return dq.reshape(shape), dk.reshape(shape), dv.reshape(shape)


def backward_rope(q_rot, k_rot, v, o, lse, do, *, causal, rope_base=10000.0, b=256, m=256,
                  r=8, recursion_base=4096, seed=0, workspace=None, cos_sin=None):
    """Gradients (dq, dk, dv) for a forward_rope call: dq and dk are those of
    the rows before their rotary embedding. q_rot and k_rot are the rotated
    rows forward_rope returned (return_rotated=True)."""
    shape, q, k, v, o, lse, do = _grad_inputs(q_rot, k_rot, v, o, lse, do)
    H, n, d = q.shape
    dt = _dtype_code(q)
    tab = _check_table(cos_sin if cos_sin is not None else
                       rope_device_table(n, d, rope_base, q.device), n, d, q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nb = backward_workspace_bytes(n, d, H, causal=causal, b=b, m=m, r=r,
                                  recursion_base=recursion_base, dtype=dt)
    ws = _workspace(workspace, nb, q)
    _call(q, lib().hyperattn_backward_rope, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
          _ptr(do), _ptr(tab), tab.shape[0], _ptr(dq), _ptr(dk), _ptr(dv), n, d, H, int(causal),
          b, m, recursion_base, r, seed, dt, _ptr(ws), ws.numel())
    return dq.reshape(shape), dk.reshape(shape), dv.reshape(shape)


def exact_backward(q, k, v, o, lse, do, *, causal=False):
    """Gradients (dq, dk, dv) of exact attention (the library's own kernels)."""
    shape, q, k, v, o, lse, do = _grad_inputs(q, k, v, o, lse, do)
    H, n, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = alloc_workspace(lib().exact_attention_backward_workspace_bytes(n, H), q.device)
    _call(q, lib().exact_attention_backward, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
          _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), n, d, H, int(causal), _dtype_code(q), _ptr(ws),
          ws.numel())
    return dq.reshape(shape), dk.reshape(shape), dv.reshape(shape)


class HyperAttentionFunction(torch.autograd.Function):
    """torch.autograd wrapper: forward and backward both run in the library.

    HyperAttentionFunction.apply(q, k, v, causal, b, m, r, recursion_base, seed).
    """

    @staticmethod
    def forward(ctx, q, k, v, causal, b, m, r, recursion_base, seed):
        o, lse = forward(q, k, v, causal=causal, b=b, m=m, r=r, recursion_base=recursion_base,
                         seed=seed, return_lse=True)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = dict(causal=causal, b=b, m=m, r=r, recursion_base=recursion_base, seed=seed)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = backward(q, k, v, o, lse, do.contiguous(), **ctx.args)
        return dq, dk, dv, None, None, None, None, None, None


class HyperAttentionRopeFunction(torch.autograd.Function):
    """torch.autograd wrapper of forward_rope (rotary embedding on the device)
    and backward_rope. HyperAttentionRopeFunction.apply(q, k, v, causal, b, m,
    r, recursion_base, seed, rope_base) with q and k before rotation."""

    @staticmethod
    def forward(ctx, q, k, v, causal, b, m, r, recursion_base, seed, rope_base):
        o, lse, qr, kr = forward_rope(q, k, v, causal=causal, rope_base=rope_base, b=b, m=m,
                                      r=r, recursion_base=recursion_base, seed=seed,
                                      return_lse=True, return_rotated=True)
        ctx.save_for_backward(qr, kr, v, o, lse)
        ctx.args = dict(causal=causal, b=b, m=m, r=r, recursion_base=recursion_base, seed=seed,
                        rope_base=rope_base)
        return o

    @staticmethod
    def backward(ctx, do):
        qr, kr, v, o, lse = ctx.saved_tensors
        dq, dk, dv = backward_rope(qr, kr, v, o, lse, do.contiguous(), **ctx.args)
        return dq, dk, dv, None, None, None, None, None, None, None


def rowsum_estimate(q, k, *, b=256, m=256, r=8, seed=0):
    """log d~ per row (Algorithm 2, non-causal)."""
    shape, q, k, _ = _qkv(q, k)
    H, n, d = q.shape
    dt = _dtype_code(q)
    out = torch.empty((H, n), dtype=torch.float32, device=q.device)
    nb = workspace_bytes(n, d, H, causal=False, b=b, m=m, r=r, recursion_base=1, dtype=dt)
    ws = alloc_workspace(nb, q.device)
    _call(q, lib().rowsum_estimate, _ptr(q), _ptr(k), n, d, H, b, m, r, seed, dt, _ptr(out),
          _ptr(ws), ws.numel())
    return out.reshape(shape[:-1])


def sortlsh_hash(x, *, r=8, seed=0, with_perm=False):
    """Hash codes [heads, n] uint8 (and the stable sort permutation if asked)."""
    shape = x.shape
    x = _fold(x, "x")
    H, n, d = x.shape
    codes = torch.empty((H, n), dtype=torch.uint8, device=x.device)
    perm = torch.empty((H, n), dtype=torch.int32, device=x.device) if with_perm else None
    nb = lib().sortlsh_hash_workspace_bytes(n, d, H, r, int(with_perm))
    if nb == 0 and _lib.last_error():
        raise _lib.HyperAttnError(-2, _lib.last_error())
    ws = alloc_workspace(nb, x.device)
    _call(x, lib().sortlsh_hash, _ptr(x), n, d, H, r, seed, _dtype_code(x), _ptr(codes),
          _ptr(perm), _ptr(ws), ws.numel())
    codes = codes.reshape(shape[:-1])
    return (codes, perm.reshape(shape[:-1])) if with_perm else codes


def hyperplanes(seed, heads, r, d):
    """The hash's Gaussian hyperplanes [heads, r, d] (host computation)."""
    G = np.empty((heads, r, d), dtype=np.float32)
    check(lib().sortlsh_hyperplanes(seed, heads, r, d,
                                    G.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
    return G


def gaussians(a, b):
    """The library's binary64 Box-Muller normals of the uint64 draws a and b."""
    a = np.ascontiguousarray(a, dtype=np.uint64)
    b = np.ascontiguousarray(b, dtype=np.uint64)
    if a.shape != b.shape:
        raise ValueError("a and b must have the same shape")
    out = np.empty(a.shape, dtype=np.float64)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    check(lib().sortlsh_gaussians(a.ctypes.data_as(u64p), b.ctypes.data_as(u64p), a.size,
                                  out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))))
    return out


_ARTIFACT_DTYPES = {"CODES_Q": np.uint8, "CODES_K": np.uint8, "VNORM_W": np.uint64,
                    "VNORM_P": np.uint64, "V_W": np.float32}


def debug_artifacts(q, k, v, *, causal, b=256, m=256, r=8, recursion_base=4096, seed=0,
                    workspace=None):
    """hyperattn_debug_artifacts: {region: host numpy array} of the forward
    pass's codes, V-norm weights and prefix sums, sorted orders and sample
    lists (flat, in the layout of workspace_layout)."""
    _, q, k, v = _qkv(q, k, v)
    H, n, d = q.shape
    dt = _dtype_code(q)
    kw = dict(causal=causal, b=b, m=m, r=r, recursion_base=recursion_base, dtype=dt)
    layout = workspace_layout(n, d, H, **kw)
    ws = _workspace(workspace, workspace_bytes(n, d, H, **kw), q)
    arrays, st = {}, _lib.HaArtifacts()
    for field, region in _lib.ARTIFACT_FIELDS:
        nbytes = layout[region][1]
        a = np.zeros(nbytes // np.dtype(_ARTIFACT_DTYPES.get(region, np.int32)).itemsize,
                     dtype=_ARTIFACT_DTYPES.get(region, np.int32))
        arrays[region] = a
        setattr(st, field, a.ctypes.data if a.size else None)
    _call(q, lib().hyperattn_debug_artifacts, _ptr(q), _ptr(k), _ptr(v), n, d, H, int(causal), b,
          m, recursion_base, r, seed, dt, _ptr(ws), ws.numel(), after=(ctypes.byref(st),))
    return arrays


def workspace_layout(n, d, heads, *, causal, b, m, r=8, recursion_base=4096, dtype=HA_BF16):
    """{region: (offset, bytes)} of hyperattn_forward's workspace."""
    off = (ctypes.c_int64 * len(_lib.WS_REGIONS))()
    nb = (ctypes.c_int64 * len(_lib.WS_REGIONS))()
    check(lib().hyperattn_workspace_layout(n, d, heads, int(causal), b, m, recursion_base, r,
                                           dtype, off, nb))
    return {name: (off[i], nb[i]) for i, name in enumerate(_lib.WS_REGIONS)}


class KernelTimer:
    """Per-kernel durations from hipEvents the library records around launches
    (stats: name -> (launches, total ms); groups: name -> work-groups launched)."""

    def __enter__(self):
        L = lib()
        check(L.hyperattn_profile_collect())
        check(L.hyperattn_profile_reset())
        check(L.hyperattn_profile_enable(1))
        return self

    def __exit__(self, *exc):
        L = lib()
        check(L.hyperattn_profile_enable(0))
        check(L.hyperattn_profile_collect())
        self.stats, self.groups = {}, {}
        for i in range(L.hyperattn_profile_count()):
            name = L.hyperattn_profile_name(i).decode()
            launches = L.hyperattn_profile_launches(i)
            if launches:
                self.stats[name] = (launches, L.hyperattn_profile_total_ms(i))
                self.groups[name] = L.hyperattn_profile_groups(i)
        return False
