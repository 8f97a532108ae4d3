"""Loads libmla_decode.so and declares its C ABI (include/mla_decode.h,
include/mla_decode_fp8.h, include/mla_kv_append.h, include/mla_absorb.h,
include/mla_mha.h).

torch is imported first on purpose: torch ships its own HIP runtime with the
same soname as /opt/rocm's, so loading the library after torch binds it to
the runtime torch already uses, and torch's streams are valid handles for it.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must be loaded before the HIP library)

# MLA_DECODE_LIB names another build of the same library (the host-sanitized
# one the sanitizer tests load); by default the library beside this file.
LIB_PATH = os.environ.get("MLA_DECODE_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                            "libmla_decode.so")

_c_int = ctypes.c_int
_c_size = ctypes.c_size_t
_c_float = ctypes.c_float
_c_ptr = ctypes.c_void_p

# name -> (restype, argtypes); every symbol the header declares
SIGNATURES = {
    "mla_status_string": (ctypes.c_char_p, [_c_int]),
    "mla_abi_version": (_c_int, []),
    "mla_default_num_partitions": (_c_int, [_c_int, _c_int]),
    "mla_metadata_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "mla_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "mla_get_split_metadata": (_c_int, [_c_ptr, _c_int, _c_int, _c_int, _c_int, _c_ptr, _c_size, _c_ptr]),
    "mla_get_split_metadata_fp8": (_c_int, [_c_ptr, _c_int, _c_int, _c_int, _c_int, _c_ptr, _c_size, _c_ptr]),
    "mla_get_split_metadata_host": (_c_int, [_c_ptr, _c_int, _c_int, _c_int, _c_int, _c_ptr, _c_size]),
    "mla_check_metadata_host": (_c_int, [_c_ptr, _c_size, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "mla_decode_fwd": (_c_int, [_c_ptr, _c_ptr, _c_ptr, _c_int, _c_ptr, _c_int, _c_int, _c_int, _c_int,
                                _c_float, _c_int, _c_ptr, _c_int, _c_ptr, _c_size, _c_ptr, _c_ptr, _c_ptr]),
    "mla_kv_append": (_c_int, [_c_ptr, _c_int, _c_int, _c_ptr, _c_ptr, _c_int, _c_ptr, _c_int, _c_ptr, _c_ptr]),
    "mla_kv_append_fp8": (_c_int, [_c_ptr, _c_int, _c_int, _c_ptr, _c_ptr, _c_int, _c_ptr, _c_int, _c_ptr,
                                   _c_ptr]),
    "mla_absorb_q": (_c_int, [_c_ptr, _c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_ptr, _c_ptr]),
    "mla_absorb_o": (_c_int, [_c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_ptr, _c_ptr]),
    "mla_decode_fwd_fp8": (_c_int, [_c_ptr, _c_ptr, _c_ptr, _c_int, _c_ptr, _c_int, _c_int, _c_int, _c_int,
                                    _c_float, _c_int, _c_ptr, _c_int, _c_ptr, _c_size, _c_ptr, _c_ptr, _c_ptr]),
    "mla_mha_decode_fwd": (_c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int, _c_ptr, _c_int, _c_int, _c_int, _c_int,
                                    _c_int, _c_float, _c_int, _c_ptr, _c_ptr, _c_ptr]),
    "mla_set_plan_override": (_c_int, [_c_int, _c_int]),
    "mla_check_decode_inputs": (_c_int, [_c_ptr, _c_int, _c_ptr, _c_int, _c_int, _c_ptr, _c_ptr]),
    "mla_decode_fwd_noalloc": (_c_int, [_c_ptr, _c_ptr, _c_ptr, _c_int, _c_ptr, _c_int, _c_int, _c_int, _c_int,
                                        _c_float, _c_int, _c_ptr, _c_int, _c_ptr, _c_ptr, _c_ptr]),
    "mla_timing_enable": (_c_int, [_c_int]),
    "mla_timing_collect": (_c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(_c_int)]),
}

MLA_OK = 0
STATUS_NAMES = {
    0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED", 3: "MLA_ERR_MISALIGNED",
    4: "MLA_ERR_WORKSPACE_TOO_SMALL", 5: "MLA_ERR_HIP", 6: "MLA_ERR_SCRATCH_LIMIT",
}


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = lib().mla_status_string(status).decode()
        super().__init__(f"{what}: {msg}")


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library. Raises ImportError if it has not been built: there
    is no fallback implementation."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing; build it with `python -m mla_paged_kv_02_amd.build` "
                "(there is no fallback path)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def check(status: int, what: str) -> None:
    if status != MLA_OK:
        raise MlaError(status, what)
