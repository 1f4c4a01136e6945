"""CPU oracle for decode attention over a growing KV cache.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product package. It
shares no code with the HIP library. ``oracle.c`` holds the fp64 arithmetic
(page "MoA-Structured Decode Attention", §2 Steps I-III, eqs. (1)-(3); §5
KV-cache accumulation; §6 GQA/MQA selection); this module only marshals numpy
arrays into it and builds it with gcc when the shared object is missing.
``brute.py`` is a second, independent pure-Python implementation in 50-digit
decimal arithmetic used to pin the C code on tiny inputs.

Element type codes: 0 = fp32, 1 = bf16 (raw uint16 bits), 2 = fp8 e4m3fn
(raw uint8 codes), 3 = int8 (two's-complement codes); fp8 and int8 values are
code times the slot's scale.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

F32, BF16, FP8_E4M3FN, INT8 = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, OpenMP) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _open(path: str):
    lib = ctypes.CDLL(path)
    P, I, F, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = D
    lib.oracle_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3fn_to_f64.restype = D
    lib.oracle_int8_to_f64.argtypes = [ctypes.c_int8]
    lib.oracle_int8_to_f64.restype = D
    lib.oracle_head_f64.argtypes = [I, I, I, D, P, P, P, P, P, P, P, P, P]
    lib.oracle_head_f64.restype = I
    lib.oracle_decode_f64_traced.argtypes = [I] * 8 + [F] + [P] * 6 + [I] + [P] * 3
    lib.oracle_decode_f64_traced.restype = I
    lib.oracle_decode_multi_f64.argtypes = [I] * 9 + [F] + [P] * 6 + [I]
    lib.oracle_decode_multi_f64.restype = I
    lib.oracle_decode_lse_f64.argtypes = [I] * 9 + [F] + [P] * 7 + [I]
    lib.oracle_decode_lse_f64.restype = I
    lib.oracle_merge_lse_f64.argtypes = [I, ctypes.c_long, I, P, P, P, P]
    lib.oracle_merge_lse_f64.restype = None
    lib.oracle_kv_append.argtypes = [I] * 6 + [P] * 5
    lib.oracle_kv_append.restype = I
    return lib


@contextlib.contextmanager
def using_library(path: str):
    """Temporarily route every call to another build of oracle.c (mutation tests)."""
    global _lib
    saved = _load()
    _lib = _open(path)
    try:
        yield
    finally:
        _lib = saved


def _load():
    global _lib
    if _lib is None:
        _lib = _open(build())
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _np(x):
    """Accept numpy arrays or CPU torch tensors (raw bits for bf16 / fp8)."""
    if isinstance(x, np.ndarray) or x is None:
        return x
    import torch  # only for tensor -> numpy bit views

    t = x.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()  # fp32, int8 (two's-complement codes), int32


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return FP8_E4M3FN
    if a.dtype == np.int8:
        return INT8
    raise TypeError(f"unsupported element type {a.dtype}")


def bf16_to_f64(bits: int) -> float:
    return _load().oracle_bf16_to_f64(int(bits))


def e4m3fn_to_f64(code: int) -> float:
    return _load().oracle_e4m3fn_to_f64(int(code))


def int8_to_f64(code: int) -> float:
    return _load().oracle_int8_to_f64(int(code))


def head_f64(q, K, V, scale: float):
    """Steps I-III for one head on fp64 arrays; returns dict of s, e, a, m, Z, out."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    n, d_k = K.shape
    d_v = V.shape[1]
    assert q.shape == (d_k,) and V.shape[0] == n
    s, e, a = (np.zeros(n) for _ in range(3))
    out = np.zeros(d_v)
    m, Z = ctypes.c_double(), ctypes.c_double()
    rc = _load().oracle_head_f64(n, d_k, d_v, float(scale), _ptr(q), _ptr(K), _ptr(V),
                                 _ptr(s), _ptr(e), _ptr(a), ctypes.addressof(m),
                                 ctypes.addressof(Z), _ptr(out))
    if rc:
        raise ValueError(f"oracle_head_f64 failed ({rc})")
    return {"s": s, "e": e, "a": a, "m": m.value, "Z": Z.value, "out": out}


def decode_f64(q, k_cache, v_cache, lens, scale: float, kv_scales=None,
               nthreads: int = 0, marks: bool = False):
    """Batched GQA decode attention in fp64.

    q [B, h_q, d_k]; k_cache [B, h_kv, cap, d_k]; v_cache [B, h_kv, cap, d_v];
    lens [B] int32 (rows attended); kv_scales [B, h_kv, 2] fp32 for fp8 / int8 caches.
    Returns out [B, h_q, d_v] float64 (and the read maps when ``marks``).
    """
    q, k_cache, v_cache, lens, kv_scales = map(_np, (q, k_cache, v_cache, lens, kv_scales))
    q, k_cache, v_cache = (np.ascontiguousarray(a) for a in (q, k_cache, v_cache))
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    B, h_q, d_k = q.shape
    _, h_kv, cap, _ = k_cache.shape
    d_v = v_cache.shape[3]
    if kv_scales is not None:
        kv_scales = np.ascontiguousarray(kv_scales, dtype=np.float32)
    out = np.zeros((B, h_q, d_v), dtype=np.float64)
    qm = km = vm = None
    if marks:
        qm = np.zeros(q.shape, np.uint8)
        km = np.zeros(k_cache.shape, np.uint8)
        vm = np.zeros(v_cache.shape, np.uint8)
    rc = _load().oracle_decode_f64_traced(
        B, h_q, h_kv, d_k, d_v, cap, _dtype_code(q), _dtype_code(k_cache),
        float(np.float32(scale)), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens),
        _ptr(kv_scales), _ptr(out), int(nthreads), _ptr(qm), _ptr(km), _ptr(vm))
    if rc:
        raise ValueError(f"oracle_decode_f64 failed ({rc})")
    return (out, (qm, km, vm)) if marks else out


def decode_multi_f64(q, k_cache, v_cache, lens, scale: float, kv_scales=None, nthreads: int = 0):
    """Multi-query causal decode in fp64: q [B, T, h_q, d_k]; query t of sequence b attends
    over its first lens[b] - T + 1 + t rows (lens[b] >= T). Returns out [B, T, h_q, d_v]."""
    q, k_cache, v_cache, lens, kv_scales = map(_np, (q, k_cache, v_cache, lens, kv_scales))
    q, k_cache, v_cache = (np.ascontiguousarray(a) for a in (q, k_cache, v_cache))
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    B, T, h_q, d_k = q.shape
    _, h_kv, cap, _ = k_cache.shape
    d_v = v_cache.shape[3]
    if kv_scales is not None:
        kv_scales = np.ascontiguousarray(kv_scales, dtype=np.float32)
    out = np.zeros((B, T, h_q, d_v), dtype=np.float64)
    rc = _load().oracle_decode_multi_f64(
        B, T, h_q, h_kv, d_k, d_v, cap, _dtype_code(q), _dtype_code(k_cache),
        float(np.float32(scale)), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens),
        _ptr(kv_scales), _ptr(out), int(nthreads))
    if rc:
        raise ValueError(f"oracle_decode_multi_f64 failed ({rc})")
    return out


def decode_lse_f64(q, k_cache, v_cache, lens, scale: float, kv_scales=None, nthreads: int = 0):
    """Decode attention over one shard of the rows, with each query row's log-sum-exp
    ln sum_l exp(s[l]) (natural log). q [B, h_q, d_k] or [B, T, h_q, d_k] (T query rows,
    causal over this cache's rows); lens[b] = 0 allowed (out 0, lse -inf).
    Returns (out [..., d_v], lse [...]) float64, shaped like q."""
    q, k_cache, v_cache, lens, kv_scales = map(_np, (q, k_cache, v_cache, lens, kv_scales))
    q, k_cache, v_cache = (np.ascontiguousarray(a) for a in (q, k_cache, v_cache))
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    single = q.ndim == 3
    q4 = q[:, None] if single else q
    q4 = np.ascontiguousarray(q4)
    B, T, h_q, d_k = q4.shape
    _, h_kv, cap, _ = k_cache.shape
    d_v = v_cache.shape[3]
    if kv_scales is not None:
        kv_scales = np.ascontiguousarray(kv_scales, dtype=np.float32)
    out = np.zeros((B, T, h_q, d_v), dtype=np.float64)
    lse = np.zeros((B, T, h_q), dtype=np.float64)
    rc = _load().oracle_decode_lse_f64(
        B, T, h_q, h_kv, d_k, d_v, cap, _dtype_code(q4), _dtype_code(k_cache),
        float(np.float32(scale)), _ptr(q4), _ptr(k_cache), _ptr(v_cache), _ptr(lens),
        _ptr(kv_scales), _ptr(out), _ptr(lse), int(nthreads))
    if rc:
        raise ValueError(f"oracle_decode_lse_f64 failed ({rc})")
    return (out[:, 0], lse[:, 0]) if single else (out, lse)


def merge_lse(outs, lses):
    """Merge of P results over disjoint row sets: outs [P, ..., d], lses [P, ...] ->
    (out [..., d], lse [...]) float64."""
    outs = np.ascontiguousarray(outs, dtype=np.float64)
    lses = np.ascontiguousarray(lses, dtype=np.float64)
    P, d = outs.shape[0], outs.shape[-1]
    rows_shape = outs.shape[1:-1]
    assert lses.shape == (P, *rows_shape)
    rows = int(np.prod(rows_shape)) if rows_shape else 1
    out = np.zeros((*rows_shape, d), dtype=np.float64)
    lse = np.zeros(rows_shape, dtype=np.float64)
    _load().oracle_merge_lse_f64(P, rows, d, _ptr(outs), _ptr(lses), _ptr(out), _ptr(lse))
    return out, lse


def kv_append(k_cache, v_cache, lens, k_new, v_new):
    """In-place KV-cache accumulation on numpy arrays (raw bits for bf16/fp8)."""
    for a in (k_cache, v_cache, lens, k_new, v_new):
        assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"]
    B, h_kv, cap, d_k = k_cache.shape
    d_v = v_cache.shape[3]
    assert lens.dtype == np.int32
    rc = _load().oracle_kv_append(B, h_kv, d_k, d_v, cap, _dtype_code(k_cache),
                                  _ptr(k_cache), _ptr(v_cache), _ptr(lens),
                                  _ptr(k_new), _ptr(v_new))
    if rc:
        raise ValueError("oracle_kv_append: a sequence is full or lens is out of range")
