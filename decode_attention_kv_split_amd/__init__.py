"""Split-KV decode attention for MI355X (gfx950): thin Python binding.

Every function here has the name of the C entry point it wraps (declared in
``include/decode_attn.h``) and does argument marshalling only: it checks the
torch tensors' dtypes, shapes, devices and contiguity, passes their device
pointers and torch's current HIP stream to ``libdecode_attn.so`` through
ctypes, and raises ``DecodeAttnError`` on a non-zero status. All arithmetic
runs in the library's HIP kernels; torch only provides device memory and the
stream. There is no fallback: if the library is not built, importing the
binding's functions fails.

Layouts (the same as the C ABI):
  q [B, h_q, d] ([B, T, h_q, d] for T = n_queries > 1) ; k_cache, v_cache [B, h_kv, cap, d] ;
  lens [B] int32 ;
  k_new, v_new [B, h_kv, d] ; kv_scales [B, h_kv, 2] fp32 (fp8 / int8 only) ;
  out [B, h_q, d] fp32 ([B, T, h_q, d] for T > 1).
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from ._lib import DA_BF16, DA_F32, DA_FP8_E4M3FN, DA_INT8, lib, library_path  # noqa: F401

__all__ = [
    "Desc", "DecodeAttnError", "Workspace", "da_workspace_size", "da_plan", "da_workspace_init",
    "kv_append", "decode_attn_run", "decode_attn_partial", "decode_attn_combine",
    "decode_attn_append_run", "decode_attn_append_partial", "decode_attn_append_combine",
    "decode_attn_run_static", "decode_attn_run_lse", "decode_attn_merge_lse",
    "da_read_device_error", "da_stream_read", "da_status_string", "da_last_error", "library_path",
    "DA_F32", "DA_BF16", "DA_FP8_E4M3FN", "DA_INT8", "DEV_ERR_APPEND_FULL", "DEV_ERR_LEN_RANGE",
    "FLAVOUR_AUTO", "FLAVOUR_VECTOR", "FLAVOUR_MATRIX", "PATH_AUTO", "PATH_SPLIT", "PATH_SINGLE",
]

DEV_ERR_APPEND_FULL = 1
DEV_ERR_LEN_RANGE = 2
FLAVOUR_AUTO, FLAVOUR_VECTOR, FLAVOUR_MATRIX = 0, 1, 2
PATH_AUTO, PATH_SPLIT, PATH_SINGLE = 0, 1, 2

_TORCH_CODE = {torch.float32: DA_F32, torch.bfloat16: DA_BF16, torch.float8_e4m3fn: DA_FP8_E4M3FN,
               torch.int8: DA_INT8}
_SCALED = (torch.float8_e4m3fn, torch.int8)  # caches of codes with per-slot scales


class DecodeAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {da_status_string(status)} ({status}): {da_last_error()}")


class _CDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("cap", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("block_rows", ctypes.c_int32), ("n_queries", ctypes.c_int32),
                ("flavour", ctypes.c_int32), ("path", ctypes.c_int32)]


@dataclass(frozen=True)
class Desc:
    """Problem descriptor (mirrors ``da_desc``). dtypes are torch dtypes."""
    batch: int
    h_q: int
    h_kv: int
    d: int
    cap: int
    q_dtype: torch.dtype
    kv_dtype: torch.dtype
    scale: float                # Step I's factor (1/sqrt(d) in the pages' setting), chosen by the caller
    block_rows: int = 0         # rows per workgroup at max_len; 0: one resident wave, equal shares
    n_queries: int = 1          # query rows per sequence (> 1: multi-query causal decode)
    flavour: int = 0            # FLAVOUR_AUTO, FLAVOUR_VECTOR or FLAVOUR_MATRIX
    path: int = 0               # PATH_AUTO, PATH_SPLIT or PATH_SINGLE (one-call entry points)

    def c(self) -> _CDesc:
        return _CDesc(self.batch, self.h_q, self.h_kv, self.d, self.d, self.cap,
                      _TORCH_CODE.get(self.q_dtype, -1), _TORCH_CODE.get(self.kv_dtype, -1),
                      float(self.scale), self.block_rows, self.n_queries, self.flavour, self.path)

    def rows_shape(self) -> tuple:
        """Shape of q and out: [B, h_q, d], or [B, T, h_q, d] with T = n_queries > 1."""
        if self.n_queries > 1:
            return (self.batch, self.n_queries, self.h_q, self.d)
        return (self.batch, self.h_q, self.d)


def _check(status: int, where: str) -> None:
    if status != 0:
        raise DecodeAttnError(status, where)


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str, shape, dtype, device=None) -> ctypes.c_void_p:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def da_status_string(status: int) -> str:
    return lib().da_status_string(int(status)).decode()


def da_last_error() -> str:
    return lib().da_last_error().decode()


def da_workspace_size(desc: Desc, max_len: int) -> int:
    n = ctypes.c_size_t()
    cd = desc.c()
    _check(lib().da_workspace_size(ctypes.byref(cd), int(max_len), ctypes.byref(n)), "da_workspace_size")
    return n.value


def da_plan(desc: Desc, max_len: int) -> dict:
    c, s, g, pa = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    cd = desc.c()
    _check(lib().da_plan(ctypes.byref(cd), int(max_len), ctypes.byref(c), ctypes.byref(s), ctypes.byref(g),
                         ctypes.byref(pa)), "da_plan")
    return {"rows_per_block": c.value, "n_blocks": s.value, "heads_per_block": g.value, "path": pa.value}


def da_workspace_init(ws: torch.Tensor) -> None:
    if ws.device.type != "cuda" or ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 GPU tensor")
    _check(lib().da_workspace_init(ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(ws)),
           "da_workspace_init")


class Workspace:
    """A device workspace sized for (desc, max_len), with its error word cleared."""

    def __init__(self, desc: Desc, max_len: int, device="cuda"):
        self.nbytes = da_workspace_size(desc, max_len)
        self.tensor = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        da_workspace_init(self.tensor)

    def ptr(self) -> ctypes.c_void_p:
        return ctypes.c_void_p(self.tensor.data_ptr())


def _ws(ws) -> tuple[ctypes.c_void_p, int, torch.Tensor]:
    t = ws.tensor if isinstance(ws, Workspace) else ws
    if t.device.type != "cuda" or t.dtype != torch.uint8 or not t.is_contiguous():
        raise ValueError("workspace must be a Workspace or a contiguous uint8 GPU tensor")
    return ctypes.c_void_p(t.data_ptr()), t.numel(), t


def _cache_shapes(desc: Desc):
    return (desc.batch, desc.h_kv, desc.cap, desc.d)


def kv_append(desc: Desc, k_cache, v_cache, lens, k_new, v_new, workspace=None) -> None:
    """Append one K row and one V row per (sequence, KV head) at row lens[b]; lens += 1."""
    dev = k_cache.device
    kc = _dev(k_cache, "k_cache", _cache_shapes(desc), desc.kv_dtype, dev)
    vc = _dev(v_cache, "v_cache", _cache_shapes(desc), desc.kv_dtype, dev)
    ln = _dev(lens, "lens", (desc.batch,), torch.int32, dev)
    kn = _dev(k_new, "k_new", (desc.batch, desc.h_kv, desc.d), desc.kv_dtype, dev)
    vn = _dev(v_new, "v_new", (desc.batch, desc.h_kv, desc.d), desc.kv_dtype, dev)
    wp = _ws(workspace)[0] if workspace is not None else ctypes.c_void_p(None)
    cd = desc.c()
    _check(lib().kv_append(ctypes.byref(cd), kc, vc, ln, kn, vn, wp, _stream(k_cache)), "kv_append")


def _attn_args(desc: Desc, q, k_cache, v_cache, lens, kv_scales):
    dev = q.device
    qp = _dev(q, "q", desc.rows_shape(), desc.q_dtype, dev)
    kc = _dev(k_cache, "k_cache", _cache_shapes(desc), desc.kv_dtype, dev)
    vc = _dev(v_cache, "v_cache", _cache_shapes(desc), desc.kv_dtype, dev)
    ln = _dev(lens, "lens", (desc.batch,), torch.int32, dev)
    if desc.kv_dtype in _SCALED:
        sc = _dev(kv_scales, "kv_scales", (desc.batch, desc.h_kv, 2), torch.float32, dev)
    else:
        sc = ctypes.c_void_p(None)
    return qp, kc, vc, ln, sc


def decode_attn_run(desc: Desc, q, k_cache, v_cache, lens, max_len: int, kv_scales, out, workspace) -> None:
    """out[b, h] = softmax(scale * K[b, h/g, :lens[b]] q[b, h]) V[b, h/g, :lens[b]]; with
    desc.n_queries = T > 1, out[b, t, h] attends over the first lens[b] - T + 1 + t rows."""
    qp, kc, vc, ln, sc = _attn_args(desc, q, k_cache, v_cache, lens, kv_scales)
    op = _dev(out, "out", desc.rows_shape(), torch.float32, q.device)
    wp, wn, _ = _ws(workspace)
    cd = desc.c()
    _check(lib().decode_attn_run(ctypes.byref(cd), qp, kc, vc, ln, int(max_len), sc, op, wp, wn, _stream(q)),
           "decode_attn_run")


def decode_attn_partial(desc: Desc, q, k_cache, v_cache, lens, max_len: int, kv_scales, workspace) -> None:
    """First stage: per-split (max, sum, unnormalised output) into the workspace."""
    qp, kc, vc, ln, sc = _attn_args(desc, q, k_cache, v_cache, lens, kv_scales)
    wp, wn, _ = _ws(workspace)
    cd = desc.c()
    _check(lib().decode_attn_partial(ctypes.byref(cd), qp, kc, vc, ln, int(max_len), sc, wp, wn, _stream(q)),
           "decode_attn_partial")


def decode_attn_combine(desc: Desc, lens, max_len: int, out, workspace) -> None:
    """Second stage: merge the splits by log-sum-exp weights into out."""
    ln = _dev(lens, "lens", (desc.batch,), torch.int32)
    op = _dev(out, "out", desc.rows_shape(), torch.float32, lens.device)
    wp, wn, _ = _ws(workspace)
    cd = desc.c()
    _check(lib().decode_attn_combine(ctypes.byref(cd), ln, int(max_len), op, wp, wn, _stream(out)),
           "decode_attn_combine")


def _append_args(desc: Desc, k_cache, k_new, v_new):
    dev = k_cache.device
    kn = _dev(k_new, "k_new", (desc.batch, desc.h_kv, desc.d), desc.kv_dtype, dev)
    vn = _dev(v_new, "v_new", (desc.batch, desc.h_kv, desc.d), desc.kv_dtype, dev)
    return kn, vn


def decode_attn_append_run(desc: Desc, q, k_cache, v_cache, lens, k_new, v_new, max_len: int, kv_scales, out,
                           workspace) -> None:
    """One decode step: append the new K/V rows, attend over lens + 1 rows, lens += 1."""
    qp, kc, vc, ln, sc = _attn_args(desc, q, k_cache, v_cache, lens, kv_scales)
    kn, vn = _append_args(desc, k_cache, k_new, v_new)
    op = _dev(out, "out", desc.rows_shape(), torch.float32, q.device)
    wp, wn, _ = _ws(workspace)
    cd = desc.c()
    _check(lib().decode_attn_append_run(ctypes.byref(cd), qp, kc, vc, ln, kn, vn, int(max_len), sc, op, wp, wn,
                                        _stream(q)), "decode_attn_append_run")


def decode_attn_append_partial(desc: Desc, q, k_cache, v_cache, lens, k_new, v_new, max_len: int, kv_scales,
                               workspace) -> None:
    """First stage of the fused step: append + per-split partials (lens unchanged)."""
    qp, kc, vc, ln, sc = _attn_args(desc, q, k_cache, v_cache, lens, kv_scales)
    kn, vn = _append_args(desc, k_cache, k_new, v_new)
    wp, wn, _ = _ws(workspace)
    cd = desc.c()
    _check(lib().decode_attn_append_partial(ctypes.byref(cd), qp, kc, vc, ln, kn, vn, int(max_len), sc, wp, wn,
                                            _stream(q)), "decode_attn_append_partial")


def decode_attn_append_combine(desc: Desc, lens, max_len: int, out, workspace) -> None:
    """Second stage of the fused step: merge into out, then lens += 1 where appended."""
    ln = _dev(lens, "lens", (desc.batch,), torch.int32)
    op = _dev(out, "out", desc.rows_shape(), torch.float32, lens.device)
    wp, wn, _ = _ws(workspace)
    cd = desc.c()
    _check(lib().decode_attn_append_combine(ctypes.byref(cd), ln, int(max_len), op, wp, wn, _stream(out)),
           "decode_attn_append_combine")


def decode_attn_run_static(desc: Desc, q, k_cache, v_cache, lens, max_len: int, kv_scales, out,
                           dev_err=None) -> None:
    """decode_attn_run with the partials in the library's static per-device scratch: no
    workspace, nothing allocated. dev_err: optional int32 GPU tensor of one element that
    receives the device error bits (the caller clears it)."""
    qp, kc, vc, ln, sc = _attn_args(desc, q, k_cache, v_cache, lens, kv_scales)
    op = _dev(out, "out", desc.rows_shape(), torch.float32, q.device)
    ep = _dev(dev_err, "dev_err", (1,), torch.int32, q.device) if dev_err is not None else ctypes.c_void_p(None)
    cd = desc.c()
    _check(lib().decode_attn_run_static(ctypes.byref(cd), qp, kc, vc, ln, int(max_len), sc, op, ep, _stream(q)),
           "decode_attn_run_static")


def decode_attn_run_lse(desc: Desc, q, k_cache, v_cache, lens, max_len: int, kv_scales, out, lse,
                        workspace) -> None:
    """decode_attn_run over one shard of the rows, also writing each query row's log-sum-exp
    (natural log of the sum of exp(scale * q . K[l]) over its rows) into lse, shaped like out
    without its last axis. lens[b] = 0: this shard holds no rows of sequence b (out 0,
    lse -inf, no device error)."""
    qp, kc, vc, ln, sc = _attn_args(desc, q, k_cache, v_cache, lens, kv_scales)
    op = _dev(out, "out", desc.rows_shape(), torch.float32, q.device)
    lp = _dev(lse, "lse", desc.rows_shape()[:-1], torch.float32, q.device)
    wp, wn, _ = _ws(workspace)
    cd = desc.c()
    _check(lib().decode_attn_run_lse(ctypes.byref(cd), qp, kc, vc, ln, int(max_len), sc, op, lp, wp, wn,
                                     _stream(q)), "decode_attn_run_lse")


def decode_attn_merge_lse(outs, lses, out, lse=None) -> None:
    """Merges P shard results over disjoint row sets: outs [P, *rows, d] and lses [P, *rows]
    (fp32 GPU tensors) into out [*rows, d] and, when given, lse [*rows]."""
    if not isinstance(outs, torch.Tensor) or outs.dim() < 2:
        raise ValueError("outs must be a tensor [P, ..., d]")
    P, d = outs.shape[0], outs.shape[-1]
    rows_shape = tuple(outs.shape[1:-1])
    dev = outs.device
    op_in = _dev(outs, "outs", tuple(outs.shape), torch.float32, dev)
    lp_in = _dev(lses, "lses", (P, *rows_shape), torch.float32, dev)
    op = _dev(out, "out", (*rows_shape, d), torch.float32, dev)
    lp = _dev(lse, "lse", rows_shape, torch.float32, dev) if lse is not None else ctypes.c_void_p(None)
    rows = 1
    for n in rows_shape:
        rows *= n
    _check(lib().decode_attn_merge_lse(ctypes.c_int64(rows), int(d), int(P), op_in, lp_in, op, lp, _stream(outs)),
           "decode_attn_merge_lse")


def da_stream_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Measurement helper: one plain streaming read of buf (contiguous, on the GPU) into sink
    (512 fp32 values)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    if not sink.is_cuda or sink.dtype != torch.float32 or sink.numel() < 512:
        raise ValueError("sink must be a GPU fp32 tensor of at least 512 values")
    nbytes = buf.numel() * buf.element_size()
    _check(lib().da_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                _stream(buf)), "da_stream_read")


def da_read_device_error(workspace) -> int:
    """Synchronises the current stream and returns the workspace's sticky error bits."""
    wp, _, t = _ws(workspace)
    code = ctypes.c_int32()
    _check(lib().da_read_device_error(wp, _stream(t), ctypes.byref(code)), "da_read_device_error")
    return code.value
