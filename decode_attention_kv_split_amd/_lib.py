"""Loads libdecode_attn.so (built in-tree) and declares its C signatures.

torch is imported first so that the library binds to the HIP runtime torch
already loaded (one runtime per process, shared streams and memory).
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (load order: torch's HIP runtime first)

DA_F32, DA_BF16, DA_FP8_E4M3FN, DA_INT8 = 0, 1, 2, 3

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libdecode_attn.so")
_lib = None

# name -> (restype, argtypes); the entry points of include/decode_attn.h
P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
SIGNATURES = {
    "da_workspace_size": (ctypes.c_int, [P, I32, P]),
    "da_plan": (ctypes.c_int, [P, I32, P, P, P, P]),
    "da_workspace_init": (ctypes.c_int, [P, SZ, P]),
    "kv_append": (ctypes.c_int, [P, P, P, P, P, P, P, P]),
    "decode_attn_run": (ctypes.c_int, [P, P, P, P, P, I32, P, P, P, SZ, P]),
    "decode_attn_partial": (ctypes.c_int, [P, P, P, P, P, I32, P, P, SZ, P]),
    "decode_attn_combine": (ctypes.c_int, [P, P, I32, P, P, SZ, P]),
    "decode_attn_append_run": (ctypes.c_int, [P, P, P, P, P, P, P, I32, P, P, P, SZ, P]),
    "decode_attn_append_partial": (ctypes.c_int, [P, P, P, P, P, P, P, I32, P, P, SZ, P]),
    "decode_attn_append_combine": (ctypes.c_int, [P, P, I32, P, P, SZ, P]),
    "decode_attn_run_static": (ctypes.c_int, [P, P, P, P, P, I32, P, P, P, P]),
    "decode_attn_run_lse": (ctypes.c_int, [P, P, P, P, P, I32, P, P, P, P, SZ, P]),
    "decode_attn_merge_lse": (ctypes.c_int, [ctypes.c_int64, I32, I32, P, P, P, P, P]),
    "da_stream_read": (ctypes.c_int, [P, SZ, P, P]),
    "da_read_device_error": (ctypes.c_int, [P, P, P]),
    "da_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "da_last_error": (ctypes.c_char_p, []),
}


def library_path() -> str:
    return _LIB_PATH


def load(path: str | None = None) -> ctypes.CDLL:
    path = path or _LIB_PATH
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built: run `python -m decode_attention_kv_split_amd.build` "
            "(or __graft_entry__.build()) first; there is no fallback path")
    lib_ = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib_, name)
        fn.restype = res
        fn.argtypes = args
    return lib_


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load()
    return _lib
