"""ctypes loader for libhyperattn.so (argument marshalling only).

The library is built in-tree by ``_build.build()``. There is no fallback: if
the shared library is missing, every entry point raises.
"""

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhyperattn.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "hyperattn.h")

HA_F32, HA_BF16 = 0, 1
STATUS = {0: "HA_OK", -1: "HA_ERR_NULL", -2: "HA_ERR_SHAPE", -3: "HA_ERR_UNSUPPORTED",
          -4: "HA_ERR_WORKSPACE", -5: "HA_ERR_HIP"}

_c = ctypes
_vp, _i64, _i32, _u64, _sz = _c.c_void_p, _c.c_int64, _c.c_int, _c.c_uint64, _c.c_size_t
_fp = _c.POINTER(_c.c_float)

SIGNATURES = {
    "hyperattn_forward": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32,
                                 _i32, _i32, _u64, _i32, _vp, _sz, _vp]),
    "hyperattn_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "hyperattn_forward_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                         _i32, _i32, _i32, _u64, _i32, _vp]),
    "hyperattn_noalloc_scratch_bytes": (_sz, []),
    "sortlsh_hash": (_i32, [_vp, _i64, _i32, _i32, _i32, _u64, _i32, _vp, _vp, _vp, _sz, _vp]),
    "sortlsh_hash_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32]),
    "exact_attention_forward": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                       _vp]),
    "rowsum_estimate": (_i32, [_vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _u64, _i32, _vp,
                               _vp, _sz, _vp]),
    "sortlsh_hyperplanes": (_i32, [_u64, _i32, _i32, _i32, _fp]),
    "sortlsh_gaussians": (_i32, [_c.POINTER(_u64), _c.POINTER(_u64), _i64,
                                 _c.POINTER(_c.c_double)]),
    "hyperattn_forward_rope": (_i32, [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _i32,
                                      _i32, _i32, _i32, _i32, _i32, _i32, _u64, _i32, _vp, _sz,
                                      _vp]),
    "rope_table": (_i32, [_i64, _i32, _c.c_double, _fp]),
    "hyperattn_backward": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32,
                                  _i32, _i32, _i32, _i32, _i32, _u64, _i32, _vp, _sz, _vp]),
    "hyperattn_backward_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                 _i32]),
    "hyperattn_backward_rope": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp,
                                       _i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _u64,
                                       _i32, _vp, _sz, _vp]),
    "exact_attention_backward": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32,
                                        _i32, _i32, _i32, _vp, _sz, _vp]),
    "exact_attention_backward_workspace_bytes": (_sz, [_i64, _i32]),
    "hyperattn_workspace_layout": (_i32, [_i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                          _c.POINTER(_i64), _c.POINTER(_i64)]),
    "hyperattn_debug_artifacts": (_i32, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _i32,
                                         _i32, _u64, _i32, _vp, _sz, _vp, _vp]),
    "hyperattn_last_error": (_c.c_char_p, []),
    "hyperattn_profile_enable": (_i32, [_i32]),
    "hyperattn_profile_collect": (_i32, []),
    "hyperattn_profile_reset": (_i32, []),
    "hyperattn_profile_count": (_i32, []),
    "hyperattn_profile_name": (_c.c_char_p, [_i32]),
    "hyperattn_profile_launches": (_i64, [_i32]),
    "hyperattn_profile_groups": (_i64, [_i32]),
    "hyperattn_profile_total_ms": (_c.c_double, [_i32]),
}

# struct ha_artifacts of include/hyperattn.h: host pointers, one per region
ARTIFACT_FIELDS = [("codes_q", "CODES_Q"), ("codes_k", "CODES_K"), ("vnorm_w", "VNORM_W"),
                   ("vnorm_p", "VNORM_P"), ("perm_q", "PERM_Q"), ("perm_k", "PERM_K"),
                   ("rank_k", "RANK_K"), ("u_idx", "U_IDX"), ("u_bkt", "U_BKT"),
                   ("v_idx", "V_IDX"), ("v_bkt", "V_BKT"), ("v_w", "V_W"),
                   ("node_meta", "NODE_META")]


class HaArtifacts(_c.Structure):
    _fields_ = [(name, _vp) for name, _ in ARTIFACT_FIELDS]


_LIB = None


class HyperAttnError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code


def lib():
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "approximate_softmax_attention_amd._build.build() (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def last_error():
    return lib().hyperattn_last_error().decode()


def check(code):
    if code != 0:
        raise HyperAttnError(code, last_error())
    return code


def header_functions():
    """Names of the functions include/hyperattn.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M))
                  - {"if", "defined"})


WS_REGIONS = ["CODES_Q", "CODES_K", "VNORM_A", "VNORM_W", "VNORM_P", "VNORM_BLK",
              "PERM_Q", "PERM_K", "RANK_K", "SORT_HIST",
              "U_IDX", "U_BKT", "V_IDX", "V_BKT", "V_W", "NODE_META",
              "PART_O", "PART_LSE", "SCHED", "PLANES",
              "DELTA", "PART_DQ", "PART_DK", "PART_DV",
              "SLOT_FIRST", "SLOT_NEXT", "SLOT_DK", "SLOT_DV"]
