"""The C ABI on the CPU: the library loads, exports what the header declares,
validates arguments before touching a device, sizes workspaces, and its host
hyperplanes equal the oracle's bit for bit. No GPU is needed."""

import ctypes
import os

import numpy as np
import pytest

from approximate_softmax_attention_amd import _lib

LIB = _lib.LIB_PATH

pytestmark = pytest.mark.skipif(not os.path.exists(LIB),
                                reason="libhyperattn.so not built (run __graft_entry__.build())")


def L():
    return _lib.lib()


def test_exports_every_declared_function():
    declared = _lib.header_functions()
    assert "hyperattn_forward" in declared and "sortlsh_hash" in declared
    assert "exact_attention_forward" in declared and "rowsum_estimate" in declared
    raw = ctypes.CDLL(LIB)
    for name in declared:
        assert hasattr(raw, name), name
    assert sorted(_lib.SIGNATURES) == declared


def test_library_has_gfx950_code_only():
    data = open(LIB, "rb").read()
    assert b"gfx950" in data
    for other in (b"gfx942", b"gfx90a", b"gfx1100"):
        assert other not in data


@pytest.mark.parametrize("seed,heads,r,d", [(0, 1, 8, 64), (1004, 2, 8, 128), (7, 3, 3, 64)])
def test_hyperplanes_equal_oracle(seed, heads, r, d):
    from approximate_softmax_attention_amd import api
    from oracle import sortlsh
    assert np.array_equal(api.hyperplanes(seed, heads, r, d),
                          sortlsh.hyperplanes(seed, heads, r, d))


@pytest.mark.parametrize("n,d,base", [(7, 64, 10000.0), (300, 128, 10000.0), (33, 64, 500.0)])
def test_rope_table_equals_oracle(n, d, base):
    """The host cos/sin table of the rotary embedding is the oracle's, bit for
    bit (fp64 from the C library, rounded once to fp32)."""
    from approximate_softmax_attention_amd import api
    from oracle import rope
    T = api.rope_table(n, d, base)
    c, s = rope.angle_table(n, d, base)
    assert np.array_equal(T[..., 0], c.astype(np.float32))
    assert np.array_equal(T[..., 1], s.astype(np.float32))


def test_forward_rope_validates_before_any_device_call():
    lib = L()
    p = _vp(256)
    # Q, K, V, cos_sin, rows, Q_rot, K_rot, O, lse, n, d, heads, causal, b, m, base, r, seed,
    # dtype, workspace, bytes, stream
    rc = lib.hyperattn_forward_rope(p, p, p, None, 1024, p, p, p, None, 1024, 64, 1, 0, 128, 128,
                                    4096, 8, 1, 1, p, 1 << 20, None)
    assert rc == -1 and "cos/sin" in _lib.last_error()
    rc = lib.hyperattn_forward_rope(p, p, p, p, 1000, p, p, p, None, 1024, 64, 1, 0, 128, 128,
                                    4096, 8, 1, 1, p, 1 << 20, None)
    assert rc == -2 and "1000 rows" in _lib.last_error()
    rc = lib.hyperattn_forward_rope(p, p, p, p, 1024, None, p, p, None, 1024, 64, 1, 0, 128, 128,
                                    4096, 8, 1, 1, p, 1 << 20, None)
    assert rc == -1 and "Q_rot" in _lib.last_error()
    rc = lib.rope_table(16, 96, 10000.0, None)
    assert rc == -3
    for base in (1.0, float("nan"), float("inf")):
        assert lib.rope_table(16, 64, base, None) == -3 and "rope_base" in _lib.last_error()


def test_backward_validates_before_any_device_call():
    lib = L()
    p = _vp(256)
    args = (1024, 64, 1, 0, 128, 128, 4096, 8, 1)
    need = lib.hyperattn_backward_workspace_bytes(*args[:8], 1)
    assert need > ws_bytes() > 0
    # fp32 and large m are not taken by the backward pass
    assert lib.hyperattn_backward_workspace_bytes(*args[:8], 0) == 0
    assert "bf16" in _lib.last_error()
    assert lib.hyperattn_backward_workspace_bytes(1024, 64, 1, 0, 128, 4096, 4096, 8, 1) == 0
    assert "m <=" in _lib.last_error()
    rc = lib.hyperattn_backward(p, p, p, p, None, p, p, p, p, 1024, 64, 1, 0, 128, 128, 4096, 8,
                                1, 1, p, need, None)
    assert rc == -1 and "lse" in _lib.last_error()
    rc = lib.hyperattn_backward(p, p, p, p, p, p, p, p, p, 1024, 64, 1, 0, 128, 128, 4096, 8, 1,
                                1, p, need - 1, None)
    assert rc == -4
    rc = lib.hyperattn_backward(p, p, p, p, p, p, p, p, p, 1000, 64, 1, 0, 128, 128, 4096, 8, 1,
                                1, p, need, None)
    assert rc == -2
    assert lib.hyperattn_backward(None, None, None, None, None, None, None, None, None, 0, 64,
                                  2, 1, 256, 256, 4096, 8, 1, 1, None, 0, None) == 0
    assert lib.exact_attention_backward_workspace_bytes(300, 2) == 2560 + 256
    rc = lib.exact_attention_backward(p, p, p, p, p, p, p, p, p, 300, 64, 2, 1, 0, p, 2816, None)
    assert rc == -3
    rc = lib.exact_attention_backward(p, p, p, p, p, p, p, p, p, 300, 64, 2, 1, 1, p, 2815, None)
    assert rc == -4


def test_backward_rope_validates_before_any_device_call():
    lib = L()
    p = _vp(256)
    need = lib.hyperattn_backward_workspace_bytes(1024, 64, 1, 0, 128, 128, 4096, 8, 1)
    # Q_rot, K_rot, V, O, lse, dO, cos_sin, rows, dQ, dK, dV, n, d, heads, causal, b, m, base,
    # r, seed, dtype, workspace, bytes, stream
    rc = lib.hyperattn_backward_rope(p, p, p, p, p, p, None, 1024, p, p, p, 1024, 64, 1, 0, 128,
                                     128, 4096, 8, 1, 1, p, need, None)
    assert rc == -1 and "cos/sin" in _lib.last_error()
    rc = lib.hyperattn_backward_rope(p, p, p, p, p, p, p, 512, p, p, p, 1024, 64, 1, 0, 128,
                                     128, 4096, 8, 1, 1, p, need, None)
    assert rc == -2 and "512 rows" in _lib.last_error()
    rc = lib.hyperattn_backward_rope(p, p, p, p, None, p, p, 1024, p, p, p, 1024, 64, 1, 0, 128,
                                     128, 4096, 8, 1, 1, p, need, None)
    assert rc == -1 and "lse" in _lib.last_error()
    rc = lib.hyperattn_backward_rope(p, p, p, p, p, p, p, 1024, p, p, p, 1024, 64, 1, 0, 128,
                                     128, 4096, 8, 1, 0, p, need, None)
    assert rc != 0 and "bf16" in _lib.last_error()
    # the gradients must not be written over the table
    rc = lib.hyperattn_backward_rope(p, p, p, p, _vp(1 << 30), p, _vp(3 << 24), 1024,
                                     _vp(3 << 24), _vp(4 << 24), _vp(5 << 24), 1024, 64, 1, 0,
                                     128, 128, 4096, 8, 1, 1, _vp(6 << 24), need, None)
    assert rc == -2 and "cos_sin" in _lib.last_error()
    assert lib.hyperattn_backward_rope(None, None, None, None, None, None, None, 0, None, None,
                                       None, 0, 64, 2, 1, 256, 256, 4096, 8, 1, 1, None, 0,
                                       None) == 0


def test_gaussians_equal_oracle_bit_for_bit():
    """The library's Box-Muller normals (binary64, before any rounding) are
    the oracle's bit for bit: both follow the same sequence of correctly
    rounded binary64 operations."""
    from approximate_softmax_attention_amd import api
    from oracle import gaussian
    rs = np.random.default_rng(12)
    a = rs.integers(0, 2 ** 64, 200000, dtype=np.uint64, endpoint=False)
    b = rs.integers(0, 2 ** 64, 200000, dtype=np.uint64, endpoint=False)
    # edges: u1 = 1 and u1 = 2^-53, the quadrant boundaries of u2, f next to sqrt 2
    edge_a = np.array([2 ** 64 - 1, 0, 2 ** 63, (2 ** 52) << 11, ((1 << 53) - 1) << 11],
                      dtype=np.uint64)
    edge_b = np.array([0, (1 << 50) << 11, ((1 << 50) - 1) << 11, (3 << 50) << 11,
                       ((7 << 50) + 1) << 11], dtype=np.uint64)
    a = np.concatenate([a, edge_a])
    b = np.concatenate([b, edge_b])
    got = api.gaussians(a, b)
    ref = gaussian.box_muller(a, b)
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))


def test_sortlsh_hash_workspace_holds_the_hyperplanes():
    lib = L()
    planes = 3 * 8 * 64 * 4 + 3 * 16 * 64 * 2
    assert lib.sortlsh_hash_workspace_bytes(1000, 64, 3, 8, 0) == planes
    assert lib.sortlsh_hash_workspace_bytes(1000, 64, 3, 8, 1) > planes
    assert lib.sortlsh_hash_workspace_bytes(1000, 96, 3, 8, 0) == 0
    assert "d=96" in _lib.last_error()


def test_backward_layout_regions():
    from approximate_softmax_attention_amd import api
    fwd = api.workspace_layout(8192, 128, 4, causal=1, b=256, m=256, recursion_base=1024)
    assert fwd["DELTA"][1] == 0 and fwd["SLOT_DK"][1] == 0
    # causal, 3 levels of 4096 slots per head: per-level bf16 partial
    # gradients of dQ, dK and dV on top of the forward's workspace
    need = L().hyperattn_backward_workspace_bytes(8192, 128, 4, 1, 256, 256, 1024, 8, 1)
    part = 3 * (3 * 4 * 4096 * 128 * 2)
    fwd_need = max(o + nb for o, nb in fwd.values())
    assert fwd_need + part <= need < fwd_need + 2 * part


def test_zero_hyperplanes_allowed():
    from approximate_softmax_attention_amd import api
    assert api.hyperplanes(5, 3, 0, 64).shape == (3, 0, 64)
    assert L().sortlsh_hyperplanes(5, 3, 0, 64, None) == 0


def ws_bytes(n=1024, d=64, heads=1, causal=0, b=128, m=128, base=4096, r=8, dt=1):
    return L().hyperattn_workspace_bytes(n, d, heads, causal, b, m, base, r, dt)


def test_workspace_sizes_and_validation_messages():
    assert ws_bytes() > 0
    assert ws_bytes(n=0) == 0 and _lib.last_error() == ""
    assert ws_bytes(d=96) == 0 and "d=96" in _lib.last_error()
    assert ws_bytes(r=9) == 0 and "r=9" in _lib.last_error()
    assert ws_bytes(r=-1) == 0 and "r=-1" in _lib.last_error()
    # r only changes the hyperplane area (fp32 [heads][max(r, 1)][d])
    assert ws_bytes(r=8) - ws_bytes(r=0) == 1 * 7 * 64 * 4 and ws_bytes(r=0) > 0
    assert ws_bytes(b=100) == 0 and "divide" in _lib.last_error()
    assert ws_bytes(n=96, causal=1, b=1, base=2) == 0 and "odd" in _lib.last_error()
    assert ws_bytes(m=0) == 0
    assert ws_bytes(dt=7) == 0
    # causal partial buffers scale with levels: n=2^17, base 4096 -> 5 levels
    big = ws_bytes(n=131072, d=128, heads=32, causal=1, b=256, m=256, base=4096)
    noncausal = ws_bytes(n=131072, d=128, heads=32, causal=0, b=256, m=256)
    assert big > noncausal > 0
    part = 5 * 32 * 65536 * 128 * 2
    assert big > part


def test_layout_regions_disjoint_and_aligned():
    from approximate_softmax_attention_amd import api
    for causal in (0, 1):
        lay = api.workspace_layout(8192, 128, 4, causal=causal, b=256, m=256,
                                   recursion_base=1024)
        total = ws_bytes(n=8192, d=128, heads=4, causal=causal, b=256, m=256, base=1024)
        spans = sorted((o, o + nb) for o, nb in lay.values() if nb > 0)
        for (a0, a1), (b0, _) in zip(spans, spans[1:]):
            assert a1 <= b0
        assert spans[-1][1] <= total
        assert all(o % 256 == 0 for o, nb in lay.values() if nb > 0)
        S = 8192 if not causal else 4096
        levels = 1 if not causal else 3
        assert lay["PERM_Q"][1] == levels * 4 * S * 4
        assert lay["VNORM_P"][1] == 4 * 8193 * 8
        assert (lay["PART_O"][1] > 0) == bool(causal)
        # hyperplanes: fp32 [4][8][128] (256-aligned), then bf16 [4][16][128]
        assert lay["PLANES"][1] == 4 * 8 * 128 * 4 + 4 * 16 * 128 * 2


def _vp(x):
    return ctypes.c_void_p(x)


def test_entry_points_validate_before_any_device_call():
    lib = L()
    p = _vp(256)    # never dereferenced: validation fails first
    # null pointers
    rc = lib.hyperattn_forward(None, p, p, p, None, 1024, 64, 1, 0, 128, 128, 4096, 8, 1, 1,
                               p, 1 << 20, None)
    assert rc == -1 and "NULL" in _lib.last_error()
    rc = lib.exact_attention_forward(p, None, p, p, None, 10, 64, 1, 0, 1, None)
    assert rc == -1
    # unsupported
    rc = lib.exact_attention_forward(p, p, p, p, None, 10, 80, 1, 0, 1, None)
    assert rc == -3
    rc = lib.sortlsh_hash(p, 10, 64, 1, 9, 1, 1, p, None, None, 0, None)
    assert rc == -3 and "r=9" in _lib.last_error()
    rc = lib.hyperattn_forward(p, p, p, p, None, 1024, 64, 1, 0, 128, 128, 4096, 8, 1, 5,
                               p, 1 << 20, None)
    assert rc == -3
    # shape
    rc = lib.hyperattn_forward(p, p, p, p, None, 1000, 64, 1, 0, 128, 128, 4096, 8, 1, 1,
                               p, 1 << 20, None)
    assert rc == -2 and "divide" in _lib.last_error()
    rc = lib.rowsum_estimate(p, p, 1000, 64, 1, 128, 1, 8, 1, 1, p, p, 1 << 20, None)
    assert rc == -2
    # workspace: too small, misaligned, missing
    need = ws_bytes()
    rc = lib.hyperattn_forward(p, p, p, p, None, 1024, 64, 1, 0, 128, 128, 4096, 8, 1, 1,
                               p, need - 1, None)
    assert rc == -4 and "needed" in _lib.last_error()
    rc = lib.hyperattn_forward(p, p, p, p, None, 1024, 64, 1, 0, 128, 128, 4096, 8, 1, 1,
                               _vp(512 + 8), need, None)
    assert rc == -4 and "aligned" in _lib.last_error()
    rc = lib.hyperattn_forward(p, p, p, p, None, 1024, 64, 1, 0, 128, 128, 4096, 8, 1, 1,
                               None, need, None)
    assert rc == -4
    rc = lib.sortlsh_hash(p, 5000, 64, 1, 8, 1, 1, p, p, None, 0, None)
    assert rc == -4
    rc = lib.sortlsh_hash(p, 5000, 64, 1, 8, 1, 1, p, None, p, 100, None)
    assert rc == -4 and "needed" in _lib.last_error()
    # empty problems are valid and touch nothing
    assert lib.hyperattn_forward(None, None, None, None, None, 0, 64, 4, 1, 256, 256, 4096,
                                 8, 1, 1, None, 0, None) == 0
    assert lib.exact_attention_forward(None, None, None, None, None, 0, 128, 2, 1, 1,
                                       None) == 0


def test_no_device_reports_hip_error():
    """With valid arguments the first device call fails here (no GPU): HA_ERR_HIP."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    lib = L()
    rc = lib.sortlsh_hash(_vp(256), 64, 64, 1, 8, 1, 1, _vp(1 << 20), None, _vp(1 << 24),
                          1 << 20, None)
    assert rc == -5 and _lib.last_error()


def test_outputs_must_not_overlap_inputs_or_each_other():
    """Written ranges (outputs, workspace) overlapping a read range or each
    other are refused with HA_ERR_SHAPE before anything is enqueued; inputs
    may share memory."""
    lib = L()
    t = 1024 * 64 * 2                       # one bf16 [1][1024][64] tensor
    q, k, v, o, ws = (_vp(i << 24) for i in range(1, 6))
    need = ws_bytes()
    # the forward's output over Q, over the workspace; lse inside O
    rc = lib.hyperattn_forward(q, k, v, q, None, 1024, 64, 1, 0, 128, 128, 4096, 8, 1, 1,
                               ws, need, None)
    assert rc == -2 and "O overlaps the input Q" in _lib.last_error()
    rc = lib.hyperattn_forward(q, k, v, _vp((5 << 24) + 256), None, 1024, 64, 1, 0, 128, 128,
                               4096, 8, 1, 1, ws, need, None)
    assert rc == -2 and "workspace" in _lib.last_error()
    rc = lib.hyperattn_forward(q, k, v, o, _vp((4 << 24) + t - 4), 1024, 64, 1, 0, 128, 128,
                               4096, 8, 1, 1, ws, need, None)
    assert rc == -2 and "O overlaps lse" in _lib.last_error()
    # Q, K and V may be one tensor (no error from the overlap check: the
    # call then fails at its first device call, here without a GPU)
    rc = lib.exact_attention_forward(q, q, q, _vp((1 << 24) + t), None, 1024, 64, 1, 0, 1, None)
    assert rc != -2
    rc = lib.exact_attention_forward(q, k, v, _vp((3 << 24) + 128), None, 1024, 64, 1, 0, 1,
                                     None)
    assert rc == -2 and "O overlaps the input V" in _lib.last_error()
    # backward: a gradient over dO, and two gradients in one buffer
    bneed = lib.hyperattn_backward_workspace_bytes(1024, 64, 1, 0, 128, 128, 4096, 8, 1)
    do, dq, dk, dv, lse = (_vp(i << 24) for i in range(6, 11))
    rc = lib.hyperattn_backward(q, k, v, o, lse, do, do, dk, dv, 1024, 64, 1, 0, 128, 128,
                                4096, 8, 1, 1, _vp(12 << 24), bneed, None)
    assert rc == -2 and "dQ overlaps the input dO" in _lib.last_error()
    rc = lib.exact_attention_backward(q, k, v, o, lse, do, dq, dq, dv, 1024, 64, 1, 0, 1,
                                      _vp(12 << 24), 1 << 20, None)
    assert rc == -2 and "dQ overlaps dK" in _lib.last_error()
    # hash codes written over the rows they hash
    rc = lib.sortlsh_hash(q, 1024, 64, 1, 8, 1, 1, _vp((1 << 24) + 100), None, ws, 1 << 20,
                          None)
    assert rc == -2 and "codes overlaps the input X" in _lib.last_error()


def test_profile_api_without_launches():
    lib = L()
    assert lib.hyperattn_profile_enable(1) == 0
    assert lib.hyperattn_profile_enable(0) == 0
    assert lib.hyperattn_profile_reset() == 0
    assert lib.hyperattn_profile_count() >= 0
    assert lib.hyperattn_profile_name(-1) == b""


def test_product_path_has_no_cpu_fallback():
    """The binding refuses to run without the HIP library instead of computing
    anything itself."""
    import importlib
    src = open(os.path.join(os.path.dirname(LIB), "api.py")).read()
    assert "oracle" not in src and "numpy.linalg" not in src
    mod = importlib.import_module("approximate_softmax_attention_amd._lib")
    saved = mod._LIB, mod.LIB_PATH
    try:
        mod._LIB, mod.LIB_PATH = None, "/nonexistent/libhyperattn.so"
        with pytest.raises(RuntimeError, match="missing"):
            mod.lib()
    finally:
        mod._LIB, mod.LIB_PATH = saved


def test_binding_checks_caller_buffers():
    """Caller-supplied outputs and workspaces are checked before any call: the
    library writes exactly q.numel() output elements and H * n lse values."""
    import torch
    from approximate_softmax_attention_amd import api
    q = torch.zeros(2, 8, 64, dtype=torch.bfloat16)
    api._check_buffer(None, "out", q, q.numel(), q.dtype)
    api._check_buffer(torch.empty(2, 8, 64, dtype=torch.bfloat16), "out", q, q.numel(), q.dtype)
    api._check_buffer(torch.empty(1, 2, 8, 64, dtype=torch.bfloat16), "out", q, q.numel(),
                      q.dtype)
    bad = [torch.empty(2, 8, 63, dtype=torch.bfloat16),          # too few elements
           torch.empty(2, 8, 64, dtype=torch.float32),           # wrong dtype
           torch.empty(2, 64, 8, dtype=torch.bfloat16).transpose(1, 2)]   # not contiguous
    for t in bad:
        with pytest.raises(ValueError):
            api._check_buffer(t, "out", q, q.numel(), q.dtype)
    with pytest.raises(ValueError):
        api._check_buffer(torch.empty(2, 9), "lse_out", q, 16, torch.float32)
    ws = torch.empty(4096, dtype=torch.uint8)
    assert api._workspace(ws, 4096, q) is ws
    with pytest.raises(ValueError):
        api._workspace(torch.empty(1024, dtype=torch.float32), 4096, q)


def test_oracle_and_product_never_import_each_other():
    """Static check of the separation: no module of the package imports the
    oracle, no oracle module imports the package, and bench.py touches the
    oracle only inside its CPU-baseline functions."""
    import ast
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

    def imports(tree):
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                for a in node.names:
                    yield node, a.name
            elif isinstance(node, ast.ImportFrom) and node.module:
                yield node, node.module

    pkg = os.path.join(root, "approximate_softmax_attention_amd")
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            tree = ast.parse(open(os.path.join(pkg, f)).read())
            assert not any(m.split(".")[0] == "oracle" for _, m in imports(tree)), f
    odir = os.path.join(root, "oracle")
    for f in os.listdir(odir):
        if f.endswith(".py"):
            tree = ast.parse(open(os.path.join(odir, f)).read())
            assert not any(m.split(".")[0] == "approximate_softmax_attention_amd"
                           for _, m in imports(tree)), f
    tree = ast.parse(open(os.path.join(root, "bench.py")).read())
    for fn in tree.body:
        uses = [m for _, m in imports(fn) if m.split(".")[0] == "oracle"]
        if uses:
            assert isinstance(fn, ast.FunctionDef) and fn.name.startswith("cpu_baseline"), \
                (getattr(fn, "name", None), uses)


def test_noalloc_forward_validates_before_any_device_call():
    """hyperattn_forward_noalloc refuses sizes whose workspace exceeds its
    64 MiB static scratch, and validates like hyperattn_forward, before any
    device call."""
    lib = L()
    p = _vp(256)
    assert lib.hyperattn_noalloc_scratch_bytes() == 64 << 20
    # 32 heads, n = 32768, d = 128, causal: 438 MiB of workspace
    rc = lib.hyperattn_forward_noalloc(p, p, p, p, None, 32768, 128, 32, 1, 256, 256, 4096, 8,
                                       1, 1, None)
    assert rc == -4 and "static scratch" in _lib.last_error()
    rc = lib.hyperattn_forward_noalloc(p, p, p, p, None, 1000, 64, 1, 0, 128, 128, 4096, 8, 1,
                                       1, None)
    assert rc == -2 and "divide" in _lib.last_error()
    rc = lib.hyperattn_forward_noalloc(None, p, p, p, None, 1024, 64, 1, 0, 128, 128, 4096, 8,
                                       1, 1, None)
    assert rc == -1
    assert lib.hyperattn_forward_noalloc(None, None, None, None, None, 0, 64, 2, 1, 256, 256,
                                         4096, 8, 1, 1, None) == 0
