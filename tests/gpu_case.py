"""Helpers for the GPU parity tests: run the HIP path through the binding on a
workload's seeded inputs, and compare with the CPU oracle at the stated tolerances.

Tolerances (fixed per KV element type; see the parity tests):
  fp32 cache: max_d |gpu - oracle| <= 1e-5 * max_d |oracle| for every (b, h)   (normwise relative)
  bf16 cache: |gpu - oracle| <= 2e-3 elementwise absolute
  fp8  cache: |gpu - oracle| <= 3e-2 elementwise absolute, the oracle run on the same
              dequantised values (code * slot scale)
  int8 cache: as fp8 (the codes widen exactly, as e4m3fn codes do, and the rest of the
              arithmetic is the same)

The absolute contract tolerances sit two to three orders of magnitude above what the
kernels reach, so a precision regression (a dropped low half of the split weights P, a bf16
rounding of a running sum, a wrong rescale: each about 1e-3 of the output) could hide under
them. Every comparison is therefore also held to a regression bound, REGRESSION, in the
fp32 contract's own measure (max_d |gpu - oracle| <= bound * max_d |oracle| per (b, h)),
about ten times the largest value that measure took on the GPU over the whole suite (the
measured maxima are stated beside each bound). The matrix-core paths keep about 18 bits of
each weight (bf16 hi + lo), so bf16 and fp8 sit near 2^-18 relative; int8 goes through
fp16 hi + lo (about 22 bits); the vector ALUs and fp32 are plain fp32.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import decode_attention_kv_split_amd as da
import oracle
import workloads

TOL = {"f32": ("rel", 1e-5), "bf16": ("abs", 2e-3), "fp8": ("abs", 3e-2), "int8": ("abs", 3e-2)}
# regression bounds, normwise relative per (b, h); measured maxima over the GPU suite:
# f32 9.6e-7, bf16 7.9e-6, fp8 5.6e-6, int8 1.0e-6
REGRESSION = {"f32": 1e-5, "bf16": 8e-5, "fp8": 6e-5, "int8": 1e-5}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def desc_of(w: workloads.Workload, block_rows: int = 0, path: int = da.PATH_AUTO) -> da.Desc:
    return da.Desc(w.B, w.h_q, w.h_kv, w.d, w.cap, workloads.TORCH_DTYPE[w.q_dtype],
                   workloads.TORCH_DTYPE[w.kv_dtype], w.scale, block_rows, 1, da.FLAVOUR_AUTO, path)


def to_gpu(case: dict, dev="cuda") -> dict:
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in case.items()}


def check_close(got: torch.Tensor, ref: np.ndarray, kv: str, what: str = "") -> float:
    """Assert the tolerance for the cache type and the regression bound; return the worst
    error in the tolerance's measure. With DA_ERROR_LOG set, every measure is appended to that
    file (how the regression bounds were measured)."""
    g = got.detach().cpu().double().numpy()
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    kind, tol = TOL[kv]
    err = np.abs(g - ref)
    rel = float((err.max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-300)).max())
    worst = rel if kind == "rel" else float(err.max())
    log_path = os.environ.get("DA_ERROR_LOG")
    if log_path:
        with open(log_path, "a") as f:
            f.write(f"{os.environ.get('PYTEST_CURRENT_TEST', '?').split(' ')[0]}\t{kv}\t"
                    f"{worst:.3e}\t{rel:.3e}\t{float(np.abs(ref).max()):.3e}\t{what}\n")
    assert worst <= tol, f"{what}: {kind} error {worst:.3e} exceeds {tol:.1e}"
    assert rel <= REGRESSION[kv], f"{what}: normwise relative error {rel:.3e} exceeds the regression bound {REGRESSION[kv]:.1e}"
    return worst


def run_gpu(w: workloads.Workload, c: dict, block_rows: int = 0, max_len: int | None = None,
            lens_key: str = "lens_final", path: int = da.PATH_AUTO):
    """Appends `steps` rows (if any) then attends once; returns out (GPU) and the GPU caches."""
    desc = desc_of(w, block_rows, path)
    g = to_gpu(c)
    lens = g["lens_init"].clone()
    ml = int(c["lens_final"].max()) if max_len is None else max_len
    ws = da.Workspace(desc, ml)
    for t in range(w.steps):
        da.kv_append(desc, g["k_cache"], g["v_cache"], lens, g["k_new"][t].contiguous(),
                     g["v_new"][t].contiguous(), ws)
    out = torch.empty(w.B, w.h_q, w.d, dtype=torch.float32, device="cuda")
    da.decode_attn_run(desc, g["q"], g["k_cache"], g["v_cache"], lens, ml, g["kv_scales"], out, ws)
    err = da.da_read_device_error(ws)
    return out, g, lens, err


def oracle_out(w: workloads.Workload, c: dict, lens=None, batch_index=None) -> np.ndarray:
    lens = c["lens_final"] if lens is None else lens
    if batch_index is None:
        kc, vc = _final_caches(w, c)
        return oracle.decode_f64(c["q"], kc, vc, lens, w.scale, kv_scales=c["kv_scales"])
    b = batch_index
    kc, vc = _final_caches(w, c, b)
    sc = None if c["kv_scales"] is None else c["kv_scales"][b:b + 1].contiguous()
    return oracle.decode_f64(c["q"][b:b + 1].contiguous(), kc, vc, lens[b:b + 1], w.scale, kv_scales=sc)


def _final_caches(w, c, b=None):
    """The caches after the appends, built with the oracle's own append."""
    sl = slice(None) if b is None else slice(b, b + 1)
    kc = oracle._np(c["k_cache"][sl]).copy()
    vc = oracle._np(c["v_cache"][sl]).copy()
    lens = oracle._np(c["lens_init"][sl]).astype(np.int32).copy()
    for t in range(w.steps):
        oracle.kv_append(kc, vc, lens, oracle._np(c["k_new"][t][sl]).copy(),
                         oracle._np(c["v_new"][t][sl]).copy())
    return kc, vc
