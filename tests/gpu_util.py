"""Helpers for the GPU parity tests: moving the shared seeded inputs to the
device, reading workspace regions back, and the tolerance measure.

Tolerance (max-relative error, per head): max |O - O_ref| / max |O_ref| must
be <= 1e-3 for fp32 inputs and <= 2e-2 for bf16 inputs (fp32 accumulation);
lse is compared as max |lse - lse_ref| against the same bounds (lse is an
absolute log quantity of order 1-10, so this is the stricter reading).
"""

import numpy as np

TOL = {"fp32": 1e-3, "bf16": 2e-2}


def torch_dtype(name):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


def to_dev(x, name):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        device="cuda", dtype=torch_dtype(name))


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def max_rel(O, ref):
    """Per-head max |O - ref| / max |ref| (largest over heads)."""
    O = np.asarray(O, dtype=np.float64).reshape(ref.shape[0], -1)
    R = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0], -1)
    return max(np.abs(O[h] - R[h]).max() / max(np.abs(R[h]).max(), 1e-30)
               for h in range(R.shape[0]))


def region(ws, layout, name, dtype):
    import torch  # noqa: F401
    off, nbytes = layout[name]
    raw = ws[off:off + nbytes].cpu().numpy()
    return raw.view(dtype)


def banner(msg):
    print(f"[gpu-case] {msg}", flush=True)
