"""Seeded random configurations on the GPU against the oracle.

A hundred configurations drawn from one fixed seed cover the product of the axes the directed
tests take one at a time: cache type (fp32, bf16, fp8, int8), head dimension (64, 128), group
size g (1 to 32, multiples of 4 or not), query rows per sequence T (1 to 8), batch, ragged
lengths from T to the capacity, rows per workgroup (the library's choice or small shares that
cut units into many segments), and the one-call or the two-stage form. Each must match the
oracle within its cache type's tolerance, with no device error; sixteen more at production-like
sizes (up to 16 sequences of 32768 rows) use the library's own partition; sixty more drive the
fused decode step.
"""
import random

import numpy as np

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


def draw_large_cases(n=16, seed=777):
    """Production-like sizes: up to 16 sequences of up to 32768 rows (4096 for fp32), so that
    the library's own partition (two workgroups per CU) cuts units into many segments."""
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        kv = rng.choice(["f32", "bf16", "bf16", "fp8", "int8"])
        d = rng.choice([64, 128])
        h_q, h_kv = rng.choice(GROUPS)
        T = rng.choice([1, 1, 1, 2, 4])
        B = rng.randint(1, 16)
        cap = 4096 if kv == "f32" else rng.choice([4096, 16384, 32768])
        block_rows = rng.choice([0, 0, 0, 4096])
        two_stage = rng.random() < 0.5
        cases.append((1000 + i, kv, d, h_q, h_kv, T, B, cap, block_rows, two_stage))
    return cases


LARGE_CASES = draw_large_cases()


@pytest.mark.parametrize("case", LARGE_CASES, ids=[f"L{c[0]}" for c in LARGE_CASES])
def test_random_configuration_large(case):
    test_random_configuration(case)


def draw_wide_cases(n=12, seed=4242, first=3000):
    """Batches around and beyond one wave's 64 lanes (up to 64 sequences the split kernel finds
    its first row from lengths held one per lane, beyond that through LDS; past 256 each thread
    of the workgroup takes several), with short caches so that the oracle stays quick."""
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        kv = rng.choice(["f32", "bf16", "bf16", "fp8", "int8"])
        d = rng.choice([64, 128])
        h_q, h_kv = rng.choice(GROUPS)
        T = rng.choice([1, 1, 2])
        B = rng.choice([63, 64, 65, 96, 257, 300])
        cap = rng.choice([64, 300])
        block_rows = rng.choice([0, 0, 17])
        two_stage = rng.random() < 0.5
        cases.append((first + i, kv, d, h_q, h_kv, T, B, cap, block_rows, two_stage))
    return cases


WIDE_CASES = draw_wide_cases()


@pytest.mark.parametrize("case", WIDE_CASES, ids=[f"W{c[0]}" for c in WIDE_CASES])
def test_random_configuration_wide_batch(case):
    test_random_configuration(case)


APPEND_CASES = [c for c in draw_cases(60, seed=4048)]


@pytest.mark.parametrize("case", APPEND_CASES, ids=[f"a{c[0]}" for c in APPEND_CASES])
def test_random_fused_step(case):
    """The fused decode step (one query row per sequence) on random configurations: the
    appended caches bit-exact, lengths + 1, and the output within tolerance of the oracle
    over the appended caches."""
    i, kv, d, h_q, h_kv, _, B, cap, block_rows, two_stage = case
    w = workloads.Workload("rand_append", B, h_q, h_kv, d, cap, "f32" if kv == "f32" else "bf16", kv,
                           ("uniform", 2, cap), 1, 9000 + i, workloads._inv_sqrt(d))
    c = workloads.generate(w)
    log(f"case random fused a{i}: {kv} d={d} h_q={h_q} h_kv={h_kv} B={B} cap={cap} block_rows={block_rows} "
        f"two_stage={two_stage} lens={c['lens_final'].tolist()}")
    desc = da.Desc(B, h_q, h_kv, d, cap, workloads.TORCH_DTYPE[w.q_dtype], workloads.TORCH_DTYPE[kv], w.scale,
                   block_rows)
    g = to_gpu(c)
    lens = g["lens_init"].clone()
    kn, vn = g["k_new"][0].contiguous(), g["v_new"][0].contiguous()
    ws = da.Workspace(desc, cap)
    out = torch.full(desc.rows_shape(), 5.0, device="cuda")
    if two_stage:
        da.decode_attn_append_partial(desc, g["q"], g["k_cache"], g["v_cache"], lens, kn, vn, cap, g["kv_scales"], ws)
        da.decode_attn_append_combine(desc, lens, cap, out, ws)
    else:
        da.decode_attn_append_run(desc, g["q"], g["k_cache"], g["v_cache"], lens, kn, vn, cap, g["kv_scales"], out, ws)
    assert da.da_read_device_error(ws) == 0
    assert lens.cpu().tolist() == c["lens_final"].tolist()
    kh, vh = oracle._np(c["k_cache"]).copy(), oracle._np(c["v_cache"]).copy()
    lh = c["lens_init"].numpy().astype(np.int32).copy()
    oracle.kv_append(kh, vh, lh, oracle._np(c["k_new"][0]).copy(), oracle._np(c["v_new"][0]).copy())
    for b in range(B):  # the rows the step wrote and everything before them
        L = int(lh[b])
        assert np.array_equal(oracle._np(g["k_cache"][b, :, :L].cpu()), kh[b, :, :L])
        assert np.array_equal(oracle._np(g["v_cache"][b, :, :L].cpu()), vh[b, :, :L])
    ref = oracle.decode_f64(c["q"], kh, vh, lh, w.scale, kv_scales=c["kv_scales"])
    check_close(out, ref, kv, f"a{i}")


WIDE_APPEND_CASES = draw_wide_cases(8, seed=4343, first=3100)


@pytest.mark.parametrize("case", WIDE_APPEND_CASES, ids=[f"wa{c[0]}" for c in WIDE_APPEND_CASES])
def test_random_fused_step_wide_batch(case):
    test_random_fused_step(case)


@pytest.mark.parametrize("two_stage", [False, True])
def test_fused_step_largest_batch(two_stage):
    """The fused step at the largest batch one call takes (1024 sequences: the prefix over
    lengths through LDS, four sequences per thread, and the copy of the stored lengths that the
    combine reads), appends bit-exact and the output within tolerance of the oracle."""
    test_random_fused_step((3200 + int(two_stage), "bf16", 64, 8, 2, 1, 1024, 64, 0, two_stage))
