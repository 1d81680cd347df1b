"""ctypes loader for ``libcosa.so`` (the C ABI declared in include/cosa.h).

Argument marshalling only.  Loading fails with an ImportError-like
``RuntimeError`` when the library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

c_i32 = ctypes.c_int32
c_i64 = ctypes.c_int64
c_f32 = ctypes.c_float
c_vp = ctypes.c_void_p
c_size = ctypes.c_size_t

COSA_OK = 0
COSA_ERR_INVALID_ARG = -1
COSA_ERR_UNSUPPORTED = -2
COSA_ERR_WORKSPACE = -3
COSA_ERR_HIP = -4
# bytes of the static workspace of cosa_proxy_ordered_mask_no_alloc
NO_ALLOC_SCRATCH_BYTES = 32 << 20


class CosaProblem(ctypes.Structure):
    _fields_ = [
        ("batch", c_i32),
        ("num_q_heads", c_i32),
        ("num_kv_heads", c_i32),
        ("head_dim", c_i32),
        ("q_block", c_i32),
        ("kv_block", c_i32),
        ("page_size", c_i32),
        ("max_seqlen", c_i32),
        ("max_pages_per_seq", c_i32),
        ("num_pages", c_i32),
        ("total_q", c_i64),
        ("softmax_scale", c_f32),
        ("cu_seqlens", c_vp),
        ("page_table", c_vp),
    ]


P = ctypes.POINTER(CosaProblem)

# name -> (restype, argtypes); must list every function include/cosa.h declares
SIGNATURES = {
    "cosa_abi_version": (c_i32, []),
    "cosa_status_string": (ctypes.c_char_p, [c_i32]),
    "cosa_last_error": (ctypes.c_char_p, []),
    "cosa_validate_problem": (c_i32, [P]),
    "cosa_num_q_tiles": (c_i64, [P]),
    "cosa_mask_capacity": (c_i64, [P, c_f32]),
    "cosa_kap_workspace_size": (c_size, [P]),
    "cosa_check_page_table_host": (c_i32, [P, c_vp, c_vp]),
    "cosa_proxy_ordered_mask": (c_i32, [P, c_vp, c_vp, c_f32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_i64, c_vp, c_size, c_vp]),
    "cosa_proxy_ordered_mask_top_p": (c_i32, [P, c_vp, c_vp, c_f32, c_f32, c_vp, c_vp, c_vp,
                                              c_vp, c_vp, c_vp, c_i64, c_vp, c_size, c_vp]),
    "cosa_proxy_ordered_mask_no_alloc": (c_i32, [P, c_vp, c_vp, c_f32, c_vp, c_vp, c_vp, c_vp,
                                                c_vp, c_vp, c_i64, c_vp]),
    "cosa_proxy_ordered_mask_shared_kv": (c_i32, [P, c_vp, c_vp, c_f32, c_f32, c_vp, c_vp,
                                                 c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_size,
                                                 c_vp]),
    "cosa_osk_prefill_shared_kv": (c_i32, [P, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_f32,
                                           c_vp, c_vp, c_vp, c_vp, c_vp]),
    "cosa_osk_prefill": (c_i32, [P, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_f32, c_vp, c_vp,
                                 c_vp, c_vp, c_vp]),
    "cosa_osk_prefill_delta": (c_i32, [P, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_f32, c_vp,
                                       c_vp, c_vp, c_vp, c_vp]),
    "cosa_dense_prefill": (c_i32, [P, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "cosa_sparse_prefill": (c_i32, [P, c_vp, c_vp, c_vp, c_f32, c_f32, c_vp, c_vp, c_vp, c_vp,
                                    c_i64, c_vp, c_size, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "cosa_block_mask_prefill": (c_i32, [P, c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp]),
}

_LIB = None


def load(path: str = None) -> ctypes.CDLL:
    """Load (once) and type the library; raise if it is not built.  The path
    defaults to ``$COSA_LIBRARY`` if set (an alternative build of the same
    sources), else the in-tree ``libcosa.so``."""
    global _LIB
    if path is None:
        path = os.environ.get("COSA_LIBRARY") or LIB_PATH
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m block_sparse_long_kap_amd.build` "
            "(hipcc for gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


class CosaError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        text = lib.cosa_status_string(status).decode()
        detail = lib.cosa_last_error().decode()
        super().__init__(f"{where}: {text} ({status}): {detail}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != COSA_OK:
        raise CosaError(status, where)
