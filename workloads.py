"""Seeded synthetic inputs for decode attention over a growing KV cache.

Shared by the tests, the smoke check and the benchmark; it feeds both the
HIP path and the CPU oracle and holds none of the method's arithmetic (no
scores, softmax or weighted sums): it only draws numbers and lays them out.

Draw order for one workload (a single ``torch.Generator('cpu')`` seeded with
the workload's seed):
  1. the per-sequence lengths, when they are random (uniform integers);
  2. q, shape [B, h_q, d], N(0, 1) in fp32;
  3. for each sequence b in order: K rows, shape [h_kv, L_b, d], then V rows,
     same shape, N(0, 1) in fp32, where L_b is the final attended length.
Values are then rounded to the storage type: bf16 with round-to-nearest-even
(``Tensor.to``); fp8 e4m3fn per (sequence, KV head, K or V) slot with scale
amax / 448 over the slot's rows (scale 1 when amax is 0), codes
clamp(x / scale, -448, 448) rounded to nearest even. The clamp matters: an
unclamped cast sends values above 448 to NaN. int8 is the symmetric 8-bit
counterpart with the same slots: scale amax / 127, codes
clamp(round-to-nearest-even(x / scale), -127, 127).

Of the L_b drawn rows, the first ``L_b - steps`` are in the cache at the
start and the rest are the rows that ``steps`` successive appends add. Rows
of the cache at or after the current length are filled with NaN ("poison"),
so any read past a sequence's end shows up in the output (int8 has no NaN:
its poison is the largest code, 127, which shifts the output instead).

Workloads follow the decode-attention shapes the pages discuss: the
single-head worked setting of page "MoA-Structured Decode Attention", the
Llama-3-8B (32 query / 8 KV heads) and Llama-2-70B (64 / 8) shapes and MQA
of page "Attention over the KV cache in the decode step" ("Derivation").
No weights or datasets are involved: every tensor is N(0, 1) noise of the
model's attention-layer shape.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import torch

FP8_MAX = 448.0
INT8_MAX = 127.0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    h_q: int
    h_kv: int
    d: int
    cap: int            # cache rows per (sequence, KV head)
    q_dtype: str        # "f32" | "bf16"
    kv_dtype: str       # "f32" | "bf16" | "fp8" | "int8"
    lens: tuple         # ("const", L) or ("uniform", lo, hi) inclusive: final attended lengths
    steps: int          # appends performed (the last `steps` drawn rows of each sequence)
    seed: int
    scale: float        # softmax scale as fp32 (1/sqrt(d))
    nq: int = 1         # query rows per sequence (> 1: multi-query causal decode)

    @property
    def g(self) -> int:
        return self.h_q // self.h_kv

    def resized(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _inv_sqrt(d: int) -> float:
    return float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))


WORKLOADS = {
    # single head, fp32, n 1008 -> 1024 over 16 append-then-attend steps
    "single_head_f32": Workload("single_head_f32", 1, 1, 1, 64, 1024, "f32", "f32",
                                ("const", 1024), 16, 1, _inv_sqrt(64)),
    # MHA, bf16 KV, every sequence 4096 rows
    "mha_bf16": Workload("mha_bf16", 8, 32, 32, 128, 4096, "bf16", "bf16",
                         ("const", 4096), 0, 2, _inv_sqrt(128)),
    # GQA 32q/8kv (Llama-3-8B shape), bf16, ragged lengths, one append per step
    "gqa8_bf16": Workload("gqa8_bf16", 16, 32, 8, 128, 32768, "bf16", "bf16",
                          ("uniform", 512, 32768), 1, 3, _inv_sqrt(128)),
    # MQA, long context
    "mqa_bf16": Workload("mqa_bf16", 4, 32, 1, 128, 131072, "bf16", "bf16",
                         ("const", 131072), 0, 4, _inv_sqrt(128)),
    # GQA 64q/8kv (Llama-2-70B shape), fp8 e4m3fn KV with per-slot scales
    "gqa8_fp8": Workload("gqa8_fp8", 32, 64, 8, 128, 16384, "bf16", "fp8",
                         ("const", 16384), 0, 5, _inv_sqrt(128)),
    # the same shape with symmetric int8 KV and per-slot scales
    "gqa8_int8": Workload("gqa8_int8", 32, 64, 8, 128, 16384, "bf16", "int8",
                          ("const", 16384), 0, 6, _inv_sqrt(128)),
    # the GQA shape verifying 4 speculative tokens per sequence: 4 query rows, causal over the
    # 4 newest rows (already in the cache)
    "gqa8_mq4_bf16": Workload("gqa8_mq4_bf16", 16, 32, 8, 128, 32768, "bf16", "bf16",
                              ("uniform", 512, 32768), 0, 7, _inv_sqrt(128), nq=4),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn,
               "int8": torch.int8}
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1}
POISON_BITS = {"f32": (torch.int32, 0x7FC00000), "bf16": (torch.int16, 0x7FC0),
               "fp8": (torch.uint8, 0x7F), "int8": (torch.int8, 127)}
SCALED = ("fp8", "int8")  # cache types whose values are code x per-slot scale


def _poisoned(shape, kind: str) -> torch.Tensor:
    itype, bits = POISON_BITS[kind]
    return torch.full(shape, bits, dtype=itype).view(TORCH_DTYPE[kind])


def quantize_e4m3fn(x: torch.Tensor):
    """Per-slot fp8 e4m3fn codes and scale for x [h_kv, L, d] (fp32)."""
    amax = x.abs().amax(dim=(1, 2))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).to(torch.float32)
    codes = (x / scale[:, None, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes, scale


def quantize_int8(x: torch.Tensor):
    """Per-slot symmetric int8 codes and scale for x [h_kv, L, d] (fp32)."""
    amax = x.abs().amax(dim=(1, 2))
    scale = torch.where(amax > 0, amax / INT8_MAX, torch.ones_like(amax)).to(torch.float32)
    codes = torch.round(x / scale[:, None, None]).clamp(-INT8_MAX, INT8_MAX).to(torch.int8)
    return codes, scale


def draw_lens(w: Workload, gen: torch.Generator) -> torch.Tensor:
    if w.lens[0] == "const":
        return torch.full((w.B,), int(w.lens[1]), dtype=torch.int32)
    lo, hi = int(w.lens[1]), int(w.lens[2])
    return torch.randint(lo, hi + 1, (w.B,), generator=gen, dtype=torch.int64).to(torch.int32)


def generate(w: Workload, seed: int | None = None, poison: bool = True) -> dict:
    """Draw one workload's inputs on the CPU.

    Returns a dict of CPU tensors:
      q          [B, h_q, d]                 q_dtype ([B, nq, h_q, d] when nq > 1)
      k_cache    [B, h_kv, cap, d]           kv_dtype, rows < lens_init valid
      v_cache    [B, h_kv, cap, d]
      lens_init  [B] int32                   rows in the cache before the appends
      lens_final [B] int32                   rows after `steps` appends
      k_new      [steps, B, h_kv, d]         rows appended at step t
      v_new      [steps, B, h_kv, d]
      kv_scales  [B, h_kv, 2] fp32 (K, V)    fp8 / int8 only, else None
      scale      float (fp32 value)
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed if seed is None else seed)
    lens = draw_lens(w, gen)
    if int(lens.max()) > w.cap or int(lens.min()) < max(1 + w.steps, w.nq):
        raise ValueError("lengths do not fit the cache")
    qshape = (w.B, w.h_q, w.d) if w.nq == 1 else (w.B, w.nq, w.h_q, w.d)
    q = torch.randn(qshape, generator=gen, dtype=torch.float32).to(TORCH_DTYPE[w.q_dtype])
    shape = (w.B, w.h_kv, w.cap, w.d)
    kv_t = TORCH_DTYPE[w.kv_dtype]
    if poison:
        k_cache, v_cache = _poisoned(shape, w.kv_dtype), _poisoned(shape, w.kv_dtype)
    else:
        k_cache, v_cache = torch.zeros(shape, dtype=kv_t), torch.zeros(shape, dtype=kv_t)
    k_new = torch.zeros((w.steps, w.B, w.h_kv, w.d), dtype=kv_t)
    v_new = torch.zeros((w.steps, w.B, w.h_kv, w.d), dtype=kv_t)
    kv_scales = torch.ones((w.B, w.h_kv, 2), dtype=torch.float32) if w.kv_dtype in SCALED else None
    quantize = quantize_e4m3fn if w.kv_dtype == "fp8" else quantize_int8
    lens_init = lens - w.steps
    for b in range(w.B):
        L = int(lens[b])
        k = torch.randn(w.h_kv, L, w.d, generator=gen, dtype=torch.float32)
        v = torch.randn(w.h_kv, L, w.d, generator=gen, dtype=torch.float32)
        if w.kv_dtype in SCALED:
            k, ks = quantize(k)
            v, vs = quantize(v)
            kv_scales[b, :, 0], kv_scales[b, :, 1] = ks, vs
        else:
            k, v = k.to(kv_t), v.to(kv_t)
        n0 = int(lens_init[b])
        k_cache[b, :, :n0] = k[:, :n0]
        v_cache[b, :, :n0] = v[:, :n0]
        for t in range(w.steps):
            k_new[t, b] = k[:, n0 + t]
            v_new[t, b] = v[:, n0 + t]
    return {"q": q, "k_cache": k_cache, "v_cache": v_cache,
            "lens_init": lens_init.contiguous(), "lens_final": lens.contiguous(),
            "k_new": k_new, "v_new": v_new, "kv_scales": kv_scales, "scale": w.scale}

