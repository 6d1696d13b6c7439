"""ctypes binding of libi4moe.so: the C ABI of include/i4moe.h under the same names.

Argument marshalling only -- every step of the path runs in the HIP library.  Loading fails
loudly when the library has not been built; there is no fallback implementation.
"""

from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libi4moe.so")

I4MOE_MAX_ROWS = 64
I4MOE_MAX_TOKENS = 64
I4MOE_MAX_K = 64
I4MOE_MAX_E = 1024
I4MOE_MAX_COLS = 8192
I4MOE_MAX_SLOTS = 16
I4MOE_GROUP_WORDS = 4 + 64 + 65 + 64 + 64 + 64 + 65 + 64
I4MOE_NOALLOC_SCRATCH_BYTES = 1048576 + 524288 + 43264

I4MOE_FMT_ROW, I4MOE_FMT_GROUP = 2, 4
I4MOE_DTYPE_F32, I4MOE_DTYPE_BF16 = 0, 1
I4MOE_OK, I4MOE_EINVAL, I4MOE_ENOMEM, I4MOE_EDEVICE = 0, -1, -2, -3
I4MOE_EUNSUPPORTED, I4MOE_EINJECTED, I4MOE_EPOISONED = -4, -5, -6
I4MOE_TAP_LOGITS, I4MOE_TAP_ROUTE, I4MOE_TAP_GROUP, I4MOE_TAP_H, I4MOE_TAP_Y = 1, 2, 3, 4, 5
I4MOE_K_ROUTE, I4MOE_K_DUAL, I4MOE_K_DOWN, I4MOE_K_TAKE, I4MOE_K_MFMA, I4MOE_K_PROBE, I4MOE_K_COUNT = 0, 1, 2, 3, 4, 5, 6


class i4moe_route_host(C.Structure):
    _fields_ = [("n", C.c_int32), ("idx", C.c_int32 * I4MOE_MAX_K), ("w", C.c_float * I4MOE_MAX_K)]


class i4moe_group(C.Structure):
    _fields_ = [("n_rows", C.c_int32), ("expert", C.POINTER(C.c_int32)), ("token", C.POINTER(C.c_int32)),
                ("weight", C.POINTER(C.c_float))]


class i4moe_host_tensor(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("gs", C.c_int32), ("O", C.c_int32), ("C", C.c_int32),
                ("packed", C.c_void_p), ("scales", C.c_void_p)]


class i4moe_tier_times(C.Structure):
    _fields_ = [("issue_ms", C.c_double), ("x_wait_ms", C.c_double), ("cpu_ms", C.c_double),
                ("total_ms", C.c_double), ("device_rows", C.c_int32), ("host_rows", C.c_int32)]


_ctx_p = C.c_void_p

# name -> (restype, argtypes); exactly the declarations of include/i4moe.h
SIGNATURES = {
    "i4moe_ctx_create": (C.c_int, [C.c_int, C.POINTER(_ctx_p)]),
    "i4moe_ctx_destroy": (C.c_int, [_ctx_p]),
    "i4moe_set_stream": (C.c_int, [_ctx_p, C.c_void_p]),
    "i4moe_last_error": (C.c_char_p, [_ctx_p]),
    "i4moe_upload_expert_tensor": (C.c_uint32, [_ctx_p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]),
    "i4moe_tensor_free": (C.c_int, [_ctx_p, C.c_uint32]),
    "i4moe_set_expert": (C.c_int, [_ctx_p, C.c_int, C.c_int, C.c_uint32, C.c_uint32, C.c_uint32]),
    "i4moe_upload_router": (C.c_int, [_ctx_p, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]),
    "i4moe_route": (C.c_int, [_ctx_p, C.c_int, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_float, C.c_int,
                              C.c_float, C.POINTER(i4moe_route_host)]),
    "i4moe_route_noalloc": (C.c_int, [_ctx_p, C.c_int, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_float, C.c_int,
                                      C.c_float, C.c_void_p]),
    "i4moe_expert_group_issue": (C.c_int, [_ctx_p, C.c_int, C.c_void_p, C.c_int, C.c_int, C.POINTER(i4moe_group)]),
    "i4moe_expert_group_take": (C.c_int, [_ctx_p, C.c_void_p, C.c_int]),
    "i4moe_set_shared_expert": (C.c_int, [_ctx_p, C.c_int, C.c_uint32, C.c_uint32, C.c_uint32]),
    "i4moe_upload_norm": (C.c_int, [_ctx_p, C.c_int, C.c_int, C.c_void_p, C.c_float]),
    "i4moe_rmsnorm": (C.c_int, [_ctx_p, C.c_int, C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_int, C.c_int]),
    "i4moe_shared_expert_issue": (C.c_int, [_ctx_p, C.c_int, C.c_void_p, C.c_int, C.c_int]),
    "i4moe_moe_block": (C.c_int, [_ctx_p, C.c_int, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_float, C.c_int,
                                  C.c_float]),
    "i4moe_set_host_expert": (C.c_int, [_ctx_p, C.c_int, C.c_int, C.POINTER(i4moe_host_tensor),
                                        C.POINTER(i4moe_host_tensor), C.POINTER(i4moe_host_tensor)]),
    "i4moe_tiered_issue": (C.c_int, [_ctx_p, C.c_int, C.c_void_p, C.c_int, C.c_int, C.POINTER(i4moe_route_host),
                                     C.POINTER(i4moe_tier_times)]),
    "i4moe_host_rows": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p,
                                  C.POINTER(i4moe_host_tensor), C.POINTER(i4moe_host_tensor),
                                  C.POINTER(i4moe_host_tensor), C.c_void_p, C.c_void_p, C.c_int]),
    "i4moe_host_int_path": (C.c_int, []),
    "i4moe_set_fail_after": (C.c_int, [_ctx_p, C.c_longlong]),
    "i4moe_debug_read": (C.c_int, [_ctx_p, C.c_int, C.c_int, C.c_void_p, C.c_size_t]),
    "i4moe_debug_size": (C.c_size_t, [_ctx_p, C.c_int, C.c_int]),
    "i4moe_set_profiling": (C.c_int, [_ctx_p, C.c_int]),
    "i4moe_profile_query": (C.c_int, [_ctx_p, C.c_int, C.POINTER(C.c_double), C.POINTER(C.c_longlong)]),
    "i4moe_read_probe": (C.c_int, [_ctx_p, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_int32)]),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libi4moe.so once; raises OSError naming the missing library."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"libi4moe.so not built at {path}; run __graft_entry__.build() first")
    # PyTorch-ROCm carries its own HIP runtime; load it first so that the library binds to
    # the same runtime instance as the tensors and streams it is handed.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _fn(name):
    def call(*args):
        return getattr(load(), name)(*args)
    call.__name__ = name
    return call


i4moe_ctx_create = _fn("i4moe_ctx_create")
i4moe_ctx_destroy = _fn("i4moe_ctx_destroy")
i4moe_set_stream = _fn("i4moe_set_stream")
i4moe_last_error = _fn("i4moe_last_error")
i4moe_upload_expert_tensor = _fn("i4moe_upload_expert_tensor")
i4moe_tensor_free = _fn("i4moe_tensor_free")
i4moe_set_expert = _fn("i4moe_set_expert")
i4moe_upload_router = _fn("i4moe_upload_router")
i4moe_route = _fn("i4moe_route")
i4moe_route_noalloc = _fn("i4moe_route_noalloc")
i4moe_expert_group_issue = _fn("i4moe_expert_group_issue")
i4moe_expert_group_take = _fn("i4moe_expert_group_take")
i4moe_set_shared_expert = _fn("i4moe_set_shared_expert")
i4moe_upload_norm = _fn("i4moe_upload_norm")
i4moe_rmsnorm = _fn("i4moe_rmsnorm")
i4moe_shared_expert_issue = _fn("i4moe_shared_expert_issue")
i4moe_moe_block = _fn("i4moe_moe_block")
i4moe_set_host_expert = _fn("i4moe_set_host_expert")
i4moe_tiered_issue = _fn("i4moe_tiered_issue")
i4moe_host_rows = _fn("i4moe_host_rows")
i4moe_host_int_path = _fn("i4moe_host_int_path")
i4moe_set_fail_after = _fn("i4moe_set_fail_after")
i4moe_debug_read = _fn("i4moe_debug_read")
i4moe_debug_size = _fn("i4moe_debug_size")
i4moe_set_profiling = _fn("i4moe_set_profiling")
i4moe_profile_query = _fn("i4moe_profile_query")
i4moe_read_probe = _fn("i4moe_read_probe")
