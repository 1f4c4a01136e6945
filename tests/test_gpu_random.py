"""Seeded random configurations on the GPU against the oracle.

A hundred configurations drawn from one fixed seed cover the product of the axes the directed
tests take one at a time: cache type (fp32, bf16, fp8, int8), head dimension (64, 128), group
size g (1 to 32, multiples of 4 or not), query rows per sequence T (1 to 8), batch, ragged
lengths from T to the capacity, rows per workgroup (the library's choice or small shares that
cut units into many segments), and the one-call or the two-stage form. Each must match the
oracle within its cache type's tolerance, with no device error.
"""
import random

import pytest
import torch

import decode_attention_kv_split_amd as da
import oracle
import workloads
from tests.gpu_case import check_close, log, to_gpu

pytestmark = pytest.mark.gpu

GROUPS = [(1, 1), (2, 1), (3, 1), (4, 1), (8, 8), (12, 4), (16, 2), (32, 8), (32, 1), (6, 3), (10, 2), (64, 8)]


def draw_cases(n=100, seed=2024):
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        kv = rng.choice(["f32", "bf16", "bf16", "fp8", "int8"])
        d = rng.choice([64, 128])
        h_q, h_kv = rng.choice(GROUPS)
        T = rng.choice([1, 1, 1, 2, 3, 4, 8])
        B = rng.randint(1, 6)
        cap = rng.choice([64, 300, 1000, 2500])
        block_rows = rng.choice([0, 0, 1, 17, 256])
        two_stage = rng.random() < 0.5
        cases.append((i, kv, d, h_q, h_kv, T, B, cap, block_rows, two_stage))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("case", CASES, ids=[f"r{c[0]}" for c in CASES])
def test_random_configuration(case):
    i, kv, d, h_q, h_kv, T, B, cap, block_rows, two_stage = case
    w = workloads.Workload("rand", B, h_q, h_kv, d, cap, "f32" if kv == "f32" else "bf16", kv,
                           ("uniform", T, cap), 0, 7000 + i, workloads._inv_sqrt(d), nq=T)
    c = workloads.generate(w)
    lens = c["lens_final"]
    log(f"case random r{i}: {kv} d={d} h_q={h_q} h_kv={h_kv} T={T} B={B} cap={cap} block_rows={block_rows} "
        f"two_stage={two_stage} lens={lens.tolist()}")
    desc = da.Desc(B, h_q, h_kv, d, cap, workloads.TORCH_DTYPE[w.q_dtype], workloads.TORCH_DTYPE[kv], w.scale,
                   block_rows, T)
    g = to_gpu(c)
    ml = int(lens.max())
    ws = da.Workspace(desc, ml)
    out = torch.full(desc.rows_shape(), 5.0, device="cuda")
    if two_stage:
        da.decode_attn_partial(desc, g["q"], g["k_cache"], g["v_cache"], g["lens_final"], ml, g["kv_scales"], ws)
        da.decode_attn_combine(desc, g["lens_final"], ml, out, ws)
    else:
        da.decode_attn_run(desc, g["q"], g["k_cache"], g["v_cache"], g["lens_final"], ml, g["kv_scales"], out, ws)
    assert da.da_read_device_error(ws) == 0
    q = c["q"] if T > 1 else c["q"].unsqueeze(1)
    ref = oracle.decode_multi_f64(q, oracle._np(c["k_cache"]), oracle._np(c["v_cache"]), lens, w.scale,
                                  kv_scales=c["kv_scales"])
    got = out if T > 1 else out.unsqueeze(1)
    check_close(got, ref, kv, f"r{i}")
