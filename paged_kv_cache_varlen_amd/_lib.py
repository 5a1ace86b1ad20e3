"""ctypes declarations of libpa.so (the C ABI in include/pa.h).

Loading needs only the HIP runtime shared library, not a GPU, so the symbol
table and the host-only entry points can be exercised on a CPU machine.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64
F32 = ctypes.c_float
SZ = ctypes.c_size_t
STATUS = ctypes.c_int

# name -> (restype, argtypes); every function declared in include/pa.h.
SIGNATURES = {
    "pa_abi_version": (ctypes.c_int, []),
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_write_kv": (STATUS, [P, P, I64, I64, P, I64, I32, I32, P, P, I64, P]),
    "pa_write_kv_fp8": (STATUS, [P, P, I64, I64, P, I64, I32, I32, F32, F32, P, P,
                                 I64, P]),
    "pa_attend_workspace_size": (SZ, [I32, I64, I32, I32, I32, I32, I32]),
    "pa_attend": (STATUS, [P, P, P, I64, P, I32, P, P, I32, I64, I32, I32, I32,
                           I32, I32, F32, P, P, SZ, P]),
    "pa_attend_noalloc": (STATUS, [P, P, P, I64, P, I32, P, P, I32, I64, I32, I32,
                                   I32, I32, I32, F32, P, P]),
    "pa_attend_plan": (STATUS, [P, I32, P, P, I32, I64, I32, I32, I32, I32, I32,
                                P, SZ, P]),
    "pa_attend_plan_fp8": (STATUS, [P, I32, P, P, I32, I64, I32, I32, I32, I32, I32,
                                    P, SZ, P]),
    "pa_attend_planned": (STATUS, [P, P, P, I64, P, I32, P, P, I32, I64, I32,
                                   I32, I32, I32, I32, F32, P, P, SZ, P]),
    "pa_attend_merge": (STATUS, [I32, I64, I32, I32, I32, I32, I32, P, P, SZ, P]),
    "pa_attend_fp8": (STATUS, [P, P, P, I64, P, I32, P, P, I32, I64, I32, I32, I32,
                               I32, I32, F32, F32, F32, P, P, SZ, P]),
    "pa_attend_planned_fp8": (STATUS, [P, P, P, I64, P, I32, P, P, I32, I64, I32,
                                       I32, I32, I32, I32, F32, F32, F32, P, P, SZ,
                                       P]),
    "pa_attend_cascade_workspace_size": (SZ, [I32, I64, I32, I32, I32, I32, I32]),
    "pa_attend_plan_cascade": (STATUS, [P, I32, P, P, I32, I64, I32, I32, I32, I32,
                                        I32, I32, P, SZ, P]),
    "pa_attend_planned_cascade": (STATUS, [P, P, P, I64, P, I32, P, P, I32, I64,
                                           I32, I32, I32, I32, I32, F32, P, P, SZ,
                                           P]),
    "pa_attend_planned_cascade_fp8": (STATUS, [P, P, P, I64, P, I32, P, P, I32, I64,
                                               I32, I32, I32, I32, I32, F32, F32,
                                               F32, P, P, SZ, P]),
    "pa_write_kv_plan": (STATUS, [P, P, I64, I64, P, I64, P, P, I64, P, I32, P, P,
                                  I32, I64, I32, I32, I32, I32, I32, I32, P, SZ, P]),
    "pa_write_kv_plan_fp8": (STATUS, [P, P, I64, I64, P, I64, F32, F32, P, P, I64, P,
                                      I32, P, P, I32, I64, I32, I32, I32, I32, I32,
                                      I32, P, SZ, P]),
    "pa_attend_merge_cascade": (STATUS, [I32, I64, I32, I32, I32, I32, I32, P, P, SZ,
                                         P]),
    "pa_attend_cascade": (STATUS, [P, P, P, I64, P, I32, P, P, I32, I64, I32, I32,
                                   I32, I32, I32, I32, F32, P, P, SZ, P]),
    "pa_attend_cascade_fp8": (STATUS, [P, P, P, I64, P, I32, P, P, I32, I64, I32,
                                       I32, I32, I32, I32, I32, F32, F32, F32, P, P,
                                       SZ, P]),
    "pa_validate_cascade_host": (STATUS, [P, I32, P, P, I32, I32]),
    "pa_copy_blocks": (STATUS, [P, P, I64, I32, I32, I32, P, I64, P]),
    "pa_expand_block_tables": (STATUS, [P, I32, I32, I32, P, P]),
    "pa_mla_workspace_size": (SZ, [I64, I32, I32]),
    "pa_mla_write_kv": (STATUS, [P, I64, P, I64, P, I64, P]),
    "pa_mla_decode": (STATUS, [P, P, I64, P, I32, P, P, I32, I64, I32, I32, F32, P, P, SZ,
                               P]),
    "pa_gather_kv": (STATUS, [P, P, I64, P, I32, P, P, I32, I64, I32, I32, P, P,
                              P]),
    "pa_write_kv_bs": (STATUS, [P, P, I64, I64, P, I64, I32, I32, P, P, I64, I32, P]),
    "pa_attend_bs": (STATUS, [P, P, P, I64, I32, P, I32, P, P, I32, I64, I32, I32, I32,
                              I32, I32, F32, P, P, SZ, P]),
    "pa_gather_kv_bs": (STATUS, [P, P, I64, I32, P, I32, P, P, I32, I64, I32, I32, P, P,
                                 P]),
    "pa_validate_metadata_host": (STATUS, [P, I32, P, P, I32, I64, I32, I32, I64,
                                           P, I64]),
    "pa_validate_metadata": (STATUS, [P, I32, P, P, I32, I64, I32, I32, I64, P,
                                      I64]),
}

PA_OK = 0
PA_ERR_NULL = 1
PA_ERR_SHAPE = 2
PA_ERR_UNSUPPORTED = 3
PA_ERR_WORKSPACE = 4
PA_ERR_METADATA = 5
PA_ERR_HIP = 6

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpa.so; raises if it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            "libpa.so is not built (%s); build it with "
            "`python -m paged_kv_cache_varlen_amd._build`" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


class PAError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.pa_last_error().decode()
        text = lib.pa_status_string(status).decode()
        super().__init__("%s failed: %s (%d): %s" % (where, text, status, msg))
        self.status = status


def check(status: int, where: str) -> None:
    if status != PA_OK:
        raise PAError(status, where)
