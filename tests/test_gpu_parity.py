"""Parity of the HIP path (through the C ABI) with the CPU oracle on the GPU.

Small cases span several row tiles, several splits and ragged tails; the
full-size workloads run in the launch configuration the benchmark times and
are compared over every sequence, the benchmarked fused decode step included.
Caches are NaN-poisoned past each sequence's length, so a read out of range
shows up as a non-finite output.
"""
import numpy as np
import pytest
import torch

import decode_attention_kv_split_amd as da
import oracle
import workloads
from tests.gpu_case import check_close, desc_of, log, oracle_out, run_gpu, to_gpu

pytestmark = pytest.mark.gpu


def W(**kw):
    base = dict(name="case", B=3, h_q=8, h_kv=2, d=128, cap=1500, q_dtype="bf16", kv_dtype="bf16",
                lens=("uniform", 1, 1500), steps=0, seed=11, scale=workloads._inv_sqrt(128))
    base.update(kw)
    if base["kv_dtype"] == "f32":
        base["q_dtype"] = "f32"
    base["scale"] = workloads._inv_sqrt(base["d"])
    return workloads.Workload(**base)


# ------------------------------------------------------------------ the single-head workload
@pytest.mark.parametrize("path", [da.PATH_SINGLE, da.PATH_SPLIT])
def test_single_head_f32_sixteen_append_then_attend_steps(path):
    """n 1008 -> 1024, fp32, 1e-5 relative per step; cache bit-exact afterwards (I4, I5)."""
    w = workloads.WORKLOADS["single_head_f32"]
    c = workloads.generate(w)
    log(f"case single_head_f32 B={w.B} d={w.d} path={path}")
    desc = desc_of(w, path=path)
    g = to_gpu(c)
    lens = g["lens_init"].clone()
    ws = da.Workspace(desc, w.cap)
    kc = oracle._np(c["k_cache"]).copy()
    vc = oracle._np(c["v_cache"]).copy()
    ln = c["lens_init"].numpy().copy()
    out = torch.empty(1, 1, w.d, device="cuda")
    for t in range(w.steps):
        da.kv_append(desc, g["k_cache"], g["v_cache"], lens, g["k_new"][t].contiguous(),
                     g["v_new"][t].contiguous(), ws)
        oracle.kv_append(kc, vc, ln, c["k_new"][t].numpy().copy(), c["v_new"][t].numpy().copy())
        da.decode_attn_run(desc, g["q"], g["k_cache"], g["v_cache"], lens, w.cap, None, out, ws)
        ref = oracle.decode_f64(c["q"], kc, vc, ln, w.scale)
        check_close(out, ref, "f32", f"step {t}")
    assert int(lens.item()) == 1024 and da.da_read_device_error(ws) == 0
    assert np.array_equal(g["k_cache"].cpu().numpy().view(np.uint32), kc.view(np.uint32))
    assert np.array_equal(g["v_cache"].cpu().numpy().view(np.uint32), vc.view(np.uint32))


# ------------------------------------------------------------------ small parity grid
CASES = [
    # kv, d, h_q, h_kv, lens, chunk
    ("f32", 64, 1, 1, ("uniform", 1, 1500), 256),
    ("f32", 128, 4, 2, ("uniform", 1, 1500), 0),
    ("f32", 64, 6, 3, ("uniform", 200, 1500), 512),
    ("bf16", 128, 8, 8, ("uniform", 1, 1500), 256),
    ("bf16", 128, 8, 2, ("uniform", 1, 1500), 0),
    ("bf16", 128, 32, 8, ("uniform", 1, 1500), 512),
    ("bf16", 64, 16, 2, ("uniform", 1, 1500), 256),
    ("bf16", 128, 32, 1, ("uniform", 700, 1500), 256),
    ("bf16", 128, 6, 2, ("uniform", 1, 1500), 256),
    ("bf16", 128, 5, 5, ("uniform", 1, 1500), 0),
    ("fp8", 128, 16, 2, ("uniform", 1, 1500), 256),
    ("fp8", 128, 8, 8, ("uniform", 1, 1500), 0),
    ("fp8", 64, 8, 1, ("uniform", 1, 1500), 512),
    ("int8", 128, 16, 2, ("uniform", 1, 1500), 256),
    ("int8", 128, 8, 8, ("uniform", 1, 1500), 0),
    ("int8", 64, 8, 1, ("uniform", 1, 1500), 512),
    ("int8", 128, 64, 2, ("uniform", 1, 1500), 0),
    # 16 heads per workgroup over short sequences: whole units written directly by one
    # workgroup (the merged sums must reach every lane of a head)
    ("bf16", 128, 32, 2, ("uniform", 1, 40), 0),
    ("fp8", 128, 32, 2, ("uniform", 1, 40), 0),
    ("bf16", 64, 64, 4, ("uniform", 1, 100), 0),
    # groups whose g has no factor of 4 or of 8: one head tile per group, padded to 16 or 32
    # query-row slots (each K and V row read once per group)
    ("bf16", 128, 10, 2, ("uniform", 1, 1500), 256),
    ("bf16", 128, 12, 1, ("uniform", 1, 1500), 0),
    ("bf16", 64, 21, 3, ("uniform", 1, 1500), 100),
    ("bf16", 128, 48, 2, ("uniform", 1, 1500), 0),
    ("fp8", 128, 9, 3, ("uniform", 1, 1500), 0),
    ("fp8", 64, 40, 2, ("uniform", 1, 1500), 256),
    ("int8", 128, 15, 3, ("uniform", 1, 1500), 0),
    ("int8", 64, 28, 1, ("uniform", 1, 1500), 100),
    ("fp8", 128, 80, 2, ("uniform", 1, 1500), 0),       # 40 rows: two tiles of 20
    ("bf16", 128, 74, 2, ("uniform", 1, 1500), 256),    # 37 rows: tiles of 19 and 18
    ("f32", 128, 12, 2, ("uniform", 1, 1500), 0),       # fp32, 6 rows in 8 vector-ALU slots
    ("f32", 64, 18, 1, ("uniform", 1, 1500), 200),      # fp32, 18 rows: tiles of 6
]


@pytest.mark.parametrize("path", ["split", "single"])
@pytest.mark.parametrize("kv,d,h_q,h_kv,lens,chunk", CASES)
def test_parity_small(kv, d, h_q, h_kv, lens, chunk, path):
    """Every case on both paths of decode_attn_run: the split kernel (with the case's shares)
    and the combine, and the single pass (one workgroup per sequence)."""
    w = W(kv_dtype=kv, d=d, h_q=h_q, h_kv=h_kv, lens=lens, seed=100 + CASES.index((kv, d, h_q, h_kv, lens, chunk)))
    c = workloads.generate(w)
    log(f"case {kv} d={d} h_q={h_q} h_kv={h_kv} chunk={chunk} path={path} lens={c['lens_final'].tolist()}")
    if path == "split":
        out, _, _, err = run_gpu(w, c, block_rows=chunk, path=da.PATH_SPLIT)
    else:
        out, _, _, err = run_gpu(w, c, path=da.PATH_SINGLE)
    assert err == 0
    check_close(out, oracle_out(w, c), kv)


@pytest.mark.parametrize("path", [da.PATH_SPLIT, da.PATH_SINGLE])
@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8", "int8"])
def test_parity_tile_and_split_boundaries(kv, path):
    """Lengths at 1, tile edges and split edges (+-1); f32/bf16 append their last row first."""
    edges = [1, 2, 63, 64, 65, 255, 256, 257, 511, 512, 513, 1023]
    steps = 0 if kv in workloads.SCALED else 1
    w = W(kv_dtype=kv, B=len(edges), h_q=4, h_kv=2, d=128, cap=1024, steps=steps,
          lens=("const", 1024), seed=5)
    c = workloads.generate(w)
    # cut sequence b to length L: drawn row L-1 becomes the appended row, rows >= L-steps poisoned
    for b, L in enumerate(edges):
        n0 = L - steps
        if steps:
            c["k_new"][0, b] = c["k_cache"][b, :, L - 1]
            c["v_new"][0, b] = c["v_cache"][b, :, L - 1]
        c["k_cache"][b, :, n0:] = workloads._poisoned(c["k_cache"][b, :, n0:].shape, kv)
        c["v_cache"][b, :, n0:] = workloads._poisoned(c["v_cache"][b, :, n0:].shape, kv)
    c["lens_final"] = torch.tensor(edges, dtype=torch.int32)
    c["lens_init"] = c["lens_final"] - steps
    log(f"case boundaries {kv} lens={edges}")
    out, _, _, err = run_gpu(w, c, block_rows=256 if path == da.PATH_SPLIT else 0, max_len=1024, path=path)
    assert err == 0
    check_close(out, oracle_out(w, c), kv)


@pytest.mark.parametrize("block_rows", [1, 37, 100, 1000])
def test_parity_uneven_workgroup_shares(block_rows):
    """Workgroup shares that are not multiples of a tile and cross (sequence, KV head)
    boundaries many times, including one-row sequences."""
    w = W(B=5, h_q=8, h_kv=2, cap=700, lens=("uniform", 1, 700), seed=60 + block_rows)
    c = workloads.generate(w)
    c["lens_final"][1] = 1
    c["lens_init"][1] = 1
    log(f"case block_rows={block_rows} lens={c['lens_final'].tolist()}")
    out, _, _, err = run_gpu(w, c, block_rows=block_rows)
    assert err == 0
    check_close(out, oracle_out(w, c), "bf16")


@pytest.mark.parametrize("kv,h_q", [("bf16", 8), ("fp8", 8), ("bf16", 2), ("f32", 3)])
def test_parity_more_workgroups_than_rows(kv, h_q):
    """A partition with far fewer rows than workgroups (block_rows 1 at max_len 1000, a few
    rows per sequence): most workgroups hold no rows, so a unit's segments sit on workgroups
    hundreds apart with empty shares in between, which the combine must skip. Both the
    one-call form and the two-stage form."""
    w = W(B=3, h_q=h_q, h_kv=2 if h_q % 2 == 0 else 1, cap=1000, kv_dtype=kv, lens=("const", 5), seed=77)
    c = workloads.generate(w)
    c["lens_final"] = torch.tensor([3, 1, 5], dtype=torch.int32)
    c["lens_init"] = c["lens_final"].clone()
    log(f"case sparse partition {kv} h_q={h_q} h_kv={w.h_kv} lens={c['lens_final'].tolist()}")
    out, g, lens, err = run_gpu(w, c, block_rows=1, max_len=1000)
    assert err == 0
    ref = oracle_out(w, c)
    check_close(out, ref, kv, "one call")
    desc = desc_of(w, 1)
    assert da.da_plan(desc, 1000)["n_blocks"] > 1000
    ws = da.Workspace(desc, 1000)
    two = torch.empty_like(out)
    da.decode_attn_partial(desc, g["q"], g["k_cache"], g["v_cache"], lens, 1000, g["kv_scales"], ws)
    da.decode_attn_combine(desc, lens, 1000, two, ws)
    assert da.da_read_device_error(ws) == 0
    check_close(two, ref, kv, "two stages")


@pytest.mark.parametrize("kv,d,h_q,h_kv", [("fp8", 128, 64, 8), ("bf16", 64, 64, 4), ("int8", 64, 64, 8)])
def test_parity_combine_with_several_rows_per_workgroup(kv, d, h_q, h_kv):
    """Batches with thousands of query rows, where the combine gives each workgroup several
    query rows of one (sequence, KV head, head tile); the two-stage form, so that every
    unit goes through the combine."""
    w = W(B=32, h_q=h_q, h_kv=h_kv, d=d, cap=300, kv_dtype=kv, lens=("uniform", 1, 300), seed=83)
    c = workloads.generate(w)
    log(f"case combine rows/workgroup {kv} d={d} h_q={h_q} h_kv={h_kv}")
    desc = desc_of(w)
    g = to_gpu(c)
    ws = da.Workspace(desc, 300)
    out = torch.empty(w.B, w.h_q, w.d, device="cuda")
    da.decode_attn_partial(desc, g["q"], g["k_cache"], g["v_cache"], g["lens_final"], 300, g["kv_scales"], ws)
    da.decode_attn_combine(desc, g["lens_final"], 300, out, ws)
    assert da.da_read_device_error(ws) == 0
    check_close(out, oracle_out(w, c), kv)


FLAVOUR_CASES = [
    # kv, d, h_q, h_kv: each run on the vector ALUs and on the matrix cores
    ("bf16", 128, 32, 8),   # g = 4, the GQA workload's group
    ("bf16", 64, 16, 2),    # g = 8: vector ALUs in two tiles of 4
    ("bf16", 128, 4, 4),    # g = 1: one query row in 16 matrix-core slots
    ("fp8", 128, 16, 2),
    ("int8", 64, 6, 3),     # g = 2
    ("fp8", 64, 12, 1),     # g = 12: three vector-ALU tiles
]


@pytest.mark.parametrize("kv,d,h_q,h_kv", FLAVOUR_CASES)
def test_both_flavours_match_the_oracle(kv, d, h_q, h_kv):
    """DA_FLAVOUR_VECTOR and DA_FLAVOUR_MATRIX on the same inputs: both within tolerance of
    the oracle, whatever the library would choose."""
    w = W(kv_dtype=kv, d=d, h_q=h_q, h_kv=h_kv, B=4, cap=2000, lens=("uniform", 1, 2000),
          seed=300 + FLAVOUR_CASES.index((kv, d, h_q, h_kv)))
    c = workloads.generate(w)
    ref = oracle_out(w, c)
    g = to_gpu(c)
    ml = int(c["lens_final"].max())
    for flavour in (da.FLAVOUR_VECTOR, da.FLAVOUR_MATRIX):
        desc = da.Desc(w.B, w.h_q, w.h_kv, w.d, w.cap, workloads.TORCH_DTYPE[w.q_dtype],
                       workloads.TORCH_DTYPE[kv], w.scale, 0, 1, flavour)
        log(f"case flavour {flavour} {kv} d={d} h_q={h_q} h_kv={h_kv} plan {da.da_plan(desc, ml)}")
        ws = da.Workspace(desc, ml)
        out = torch.empty(w.B, w.h_q, w.d, device="cuda")
        da.decode_attn_run(desc, g["q"], g["k_cache"], g["v_cache"], g["lens_final"], ml, g["kv_scales"], out, ws)
        assert da.da_read_device_error(ws) == 0
        check_close(out, ref, kv, f"flavour {flavour}")


@pytest.mark.parametrize("path", [da.PATH_SPLIT, da.PATH_SINGLE])
def test_invalid_lengths_between_valid_ones(path):
    """Sequences with an out-of-range length hold no rows of the partition: their output
    is zeroed and flagged, and the sequences around them are unaffected."""
    w = W(B=4, h_q=8, h_kv=2, cap=600, lens=("const", 600), seed=71)
    c = workloads.generate(w)
    desc = desc_of(w, 100 if path == da.PATH_SPLIT else 0, path)
    g = to_gpu(c)
    lens = torch.tensor([300, 0, 600, 500], dtype=torch.int32)
    ws = da.Workspace(desc, 550)
    out = torch.full((w.B, w.h_q, w.d), 3.0, device="cuda")
    da.decode_attn_run(desc, g["q"], g["k_cache"], g["v_cache"], lens.cuda(), 550, None, out, ws)
    assert da.da_read_device_error(ws) == da.DEV_ERR_LEN_RANGE
    o = out.cpu()
    assert torch.equal(o[1], torch.zeros(8, 128)) and torch.equal(o[2], torch.zeros(8, 128))
    ok = torch.tensor([300, 1, 1, 500], dtype=torch.int32)
    ref = oracle_out(w, c, lens=ok)
    check_close(o[[0, 3]], ref[[0, 3]], "bf16")


@pytest.mark.parametrize("B", [64, 65])
@pytest.mark.parametrize("h_q", [8, 2])  # g = 4: matrix cores; g = 1: vector ALUs
def test_batch_at_the_edge_of_one_wave(B, h_q):
    """64 sequences are the most that a wave holds one per lane (the prefix over lengths in
    registers); 65 go through LDS. Shares of 37 rows cross many sequences, and sequences
    without rows (length 0, or above max_len) lie between valid ones and at the end, so the
    walk skips them in both forms."""
    w = W(B=B, h_q=h_q, h_kv=2, d=64, cap=200, lens=("uniform", 1, 150), seed=300 + B + h_q)
    c = workloads.generate(w)
    lens = c["lens_final"].clone()
    lens[::7] = 0
    lens[3::11] = 190  # above max_len = 150
    lens[-2:] = 0
    valid = (lens >= 1) & (lens <= 150)
    desc = desc_of(w, 37, da.PATH_SPLIT)
    g = to_gpu(c)
    ws = da.Workspace(desc, 150)
    out = torch.full((w.B, w.h_q, w.d), 3.0, device="cuda")
    log(f"case batch {B} h_q={h_q} with empty sequences")
    da.decode_attn_run(desc, g["q"], g["k_cache"], g["v_cache"], lens.cuda(), 150, None, out, ws)
    assert da.da_read_device_error(ws) == da.DEV_ERR_LEN_RANGE
    o = out.cpu()
    assert torch.equal(o[~valid], torch.zeros(int((~valid).sum()), w.h_q, w.d))
    ref = oracle_out(w, c, lens=torch.where(valid, lens, torch.ones_like(lens)))
    idx = valid.nonzero().flatten()
    check_close(o[idx], ref[idx.numpy()], "bf16", f"B={B} h_q={h_q}")


def test_single_row_returns_that_value_row_exactly():
    """I1: with one row the softmax weight is 1 and out equals the V row (bf16 widened)."""
    w = W(B=4, h_q=8, h_kv=2, cap=300, lens=("const", 1))
    c = workloads.generate(w)
    out, _, _, err = run_gpu(w, c, max_len=1)
    assert err == 0
    expect = c["v_cache"][:, :, 0].float().repeat_interleave(w.g, dim=1)
    assert torch.equal(out.cpu(), expect)


@pytest.mark.parametrize("h_q", [1, 4])
def test_fp8_decoding_of_every_finite_code(h_q):
    """The e4m3fn decode of V: with one row per sequence out = decode(code) * v_scale, checked
    for all 254 finite codes against the oracle's decoder (v_scale = 1, exact), on both
    flavours (one query head: the vector ALUs' bit decoder; four: the matrix cores' paired
    conversion, after the LDS stage), and with every code at each of the four byte positions of
    a 32-bit word (four rotations of the code order)."""
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    for rot in range(4):
        codes = [0] * rot + finite
        codes += [0] * (512 - len(codes))
        w = W(B=4, h_q=h_q, h_kv=1, d=128, cap=64, kv_dtype="fp8", lens=("const", 1))
        c = workloads.generate(w)
        v = torch.tensor(codes, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).reshape(4, 128)
        c["v_cache"][:, 0, 0] = v
        c["kv_scales"][:] = 1.0
        out, _, _, err = run_gpu(w, c, max_len=1)
        assert err == 0
        expect = np.array([oracle.e4m3fn_to_f64(x) for x in codes]).reshape(4, 1, 128)
        assert np.array_equal(out.cpu().double().numpy(), np.repeat(expect, h_q, axis=1)), f"rotation {rot}"


def test_int8_decoding_of_every_code():
    """The in-register int8 decode: with one row per sequence out = code * v_scale, checked
    for all 256 codes against the oracle's decoder (v_scale = 1, exact), on both flavours
    (one query head per KV head: vector ALUs; four: matrix cores through the LDS stages)."""
    codes = list(range(-128, 128))
    for h_q in (1, 4):
        w = W(B=2, h_q=h_q, h_kv=1, d=128, cap=64, kv_dtype="int8", lens=("const", 1))
        c = workloads.generate(w)
        c["v_cache"][:, 0, 0] = torch.tensor(codes, dtype=torch.int8).reshape(2, 128)
        c["kv_scales"][:] = 1.0
        out, _, _, err = run_gpu(w, c, max_len=1)
        assert err == 0
        expect = np.array([oracle.int8_to_f64(x) for x in codes]).reshape(2, 1, 128)
        assert np.array_equal(out.cpu().double().numpy(), np.repeat(expect, h_q, axis=1)), f"h_q={h_q}"


@pytest.mark.parametrize("qmul", [2.0 ** -20, 2.0 ** -8, 1.0, 2.0 ** 8, 2.0 ** 17])
@pytest.mark.parametrize("d", [128, 64])
def test_int8_matrix_cores_across_query_magnitudes(qmul, d):
    """The int8 matrix-core path runs Step I in fp16 with q scaled by a power of two per head:
    queries from 2^-20 to 2^17 times N(0, 1) (beyond fp16's range at the top, in its subnormals
    at the bottom) must still match the oracle."""
    w = W(B=2, h_q=8, h_kv=1, d=d, cap=400, kv_dtype="int8", lens=("uniform", 1, 400), seed=91)
    c = workloads.generate(w)
    c["q"] = (c["q"].float() * qmul).to(torch.bfloat16)
    log(f"case int8 q x {qmul} d={d} lens={c['lens_final'].tolist()}")
    out, _, _, err = run_gpu(w, c)
    assert err == 0
    check_close(out, oracle_out(w, c), "int8")


def test_gqa_equals_mha_on_broadcast_cache():
    """I3 on the GPU: the grouped kernel equals the one-head-per-group kernel on a
    repeat_interleave'd cache, within the bf16 tolerance."""
    w = W(B=3, h_q=16, h_kv=4, cap=1200, lens=("uniform", 1, 1200), seed=31)
    c = workloads.generate(w)
    out_gqa, _, _, _ = run_gpu(w, c)
    wm = W(B=3, h_q=16, h_kv=16, cap=1200, lens=("uniform", 1, 1200), seed=31)
    cm = dict(c)
    cm["k_cache"] = c["k_cache"].repeat_interleave(w.g, dim=1).contiguous()
    cm["v_cache"] = c["v_cache"].repeat_interleave(w.g, dim=1).contiguous()
    out_mha, _, _, _ = run_gpu(wm, cm)
    assert (out_gqa - out_mha).abs().max().item() <= 2e-3
    check_close(out_gqa, oracle_out(w, c), "bf16")


def test_two_stage_path_matches_fused_run():
    """decode_attn_partial + decode_attn_combine (the split partials merged by a separate
    kernel) agree with the fused decode_attn_run and with the oracle."""
    w = W(B=4, h_q=16, h_kv=4, cap=3000, lens=("uniform", 1, 3000), seed=43)
    c = workloads.generate(w)
    desc = desc_of(w, 256)
    g = to_gpu(c)
    ml = int(c["lens_final"].max())
    ws = da.Workspace(desc, ml)
    fused = torch.empty(w.B, w.h_q, w.d, device="cuda")
    da.decode_attn_run(desc, g["q"], g["k_cache"], g["v_cache"], g["lens_final"], ml, None, fused, ws)
    two = torch.empty_like(fused)
    da.decode_attn_partial(desc, g["q"], g["k_cache"], g["v_cache"], g["lens_final"], ml, None, ws)
    da.decode_attn_combine(desc, g["lens_final"], ml, two, ws)
    assert da.da_read_device_error(ws) == 0
    assert (fused - two).abs().max().item() <= 1e-5
    check_close(two, oracle_out(w, c), "bf16")


def test_workspace_reuse_across_calls():
    """One workspace serves a sequence of calls with different lengths (single- and
    multi-split sequences): nothing from an earlier call leaks into a later one."""
    w = W(B=5, h_q=8, h_kv=2, cap=2000, lens=("const", 2000), seed=47)
    c = workloads.generate(w)
    desc = desc_of(w, 256)
    g = to_gpu(c)
    ws = da.Workspace(desc, w.cap)
    out = torch.empty(w.B, w.h_q, w.d, device="cuda")
    for lens in ([2000, 1, 256, 257, 1999], [5, 2000, 700, 256, 1], [1000, 1000, 1000, 1000, 1000]):
        lt = torch.tensor(lens, dtype=torch.int32)
        da.decode_attn_run(desc, g["q"], g["k_cache"], g["v_cache"], lt.cuda(), w.cap, None, out, ws)
        check_close(out, oracle_out(w, c, lens=lt), "bf16", f"lens {lens}")
    assert da.da_read_device_error(ws) == 0


def test_one_workspace_serves_both_paths_in_turn():
    """The two-stage entry points (split path) and decode_attn_run on the single pass, in turn on
    one workspace: the split path never touches the single pass's counters, which every single
    pass leaves at zero."""
    w = W(B=6, h_q=8, h_kv=2, d=64, cap=500, lens=("uniform", 1, 500), seed=48)
    c = workloads.generate(w)
    desc = desc_of(w)
    assert da.da_plan(desc, w.cap)["path"] == da.PATH_SINGLE
    g = to_gpu(c)
    ws = da.Workspace(desc, w.cap)
    ref = oracle_out(w, c)
    for _ in range(3):
        two = torch.empty(w.B, w.h_q, w.d, device="cuda")
        da.decode_attn_partial(desc, g["q"], g["k_cache"], g["v_cache"], g["lens_final"], w.cap, None, ws)
        da.decode_attn_combine(desc, g["lens_final"], w.cap, two, ws)
        one = torch.full_like(two, 9.0)
        da.decode_attn_run(desc, g["q"], g["k_cache"], g["v_cache"], g["lens_final"], w.cap, None, one, ws)
        assert da.da_read_device_error(ws) == 0
        check_close(two, ref, "bf16", "split path")
        check_close(one, ref, "bf16", "single pass")


def test_runs_are_bitwise_deterministic():
    w = W(B=4, h_q=32, h_kv=8, cap=3000, lens=("uniform", 1, 3000), seed=41)
    c = workloads.generate(w)
    a, _, _, _ = run_gpu(w, c, block_rows=256)
    b, _, _, _ = run_gpu(w, c, block_rows=256)
    assert torch.equal(a, b)


def test_append_is_bit_exact_over_the_whole_buffer():
    w = W(B=5, h_q=8, h_kv=4, d=128, cap=40, lens=("uniform", 3, 40), steps=3, seed=9)
    c = workloads.generate(w)
    desc = desc_of(w)
    g = to_gpu(c)
    lens = g["lens_init"].clone()
    ws = da.Workspace(desc, w.cap)
    kc = oracle._np(c["k_cache"]).copy()
    vc = oracle._np(c["v_cache"]).copy()
    ln = c["lens_init"].numpy().copy()
    for t in range(w.steps):
        da.kv_append(desc, g["k_cache"], g["v_cache"], lens, g["k_new"][t].contiguous(),
                     g["v_new"][t].contiguous(), ws)
        oracle.kv_append(kc, vc, ln, oracle._np(c["k_new"][t]).copy(), oracle._np(c["v_new"][t]).copy())
    assert np.array_equal(oracle._np(g["k_cache"].cpu()), kc)
    assert np.array_equal(oracle._np(g["v_cache"].cpu()), vc)
    assert np.array_equal(lens.cpu().numpy(), ln) and da.da_read_device_error(ws) == 0


@pytest.mark.parametrize("path", [da.PATH_SPLIT, da.PATH_SINGLE])
def test_device_errors_are_flagged_and_work_skipped(path):
    """A full sequence is not appended to; an out-of-range length gives zeros; both set bits."""
    w = W(B=2, h_q=4, h_kv=2, d=128, cap=16, lens=("const", 16), steps=0, seed=2)
    c = workloads.generate(w)
    desc = desc_of(w, path=path)
    g = to_gpu(c)
    ws = da.Workspace(desc, 16)
    lens = torch.tensor([16, 5], dtype=torch.int32, device="cuda")
    before = g["k_cache"].clone()
    row = torch.zeros(2, 2, 128, dtype=torch.bfloat16, device="cuda")
    da.kv_append(desc, g["k_cache"], g["v_cache"], lens, row, row, ws)
    assert da.da_read_device_error(ws) == da.DEV_ERR_APPEND_FULL
    assert lens.tolist() == [16, 6]
    assert torch.equal(g["k_cache"][0], before[0])
    ws2 = da.Workspace(desc, 8)
    out = torch.full((2, 4, 128), 7.0, device="cuda")
    da.decode_attn_run(desc, g["q"], g["k_cache"], g["v_cache"], lens, 8, None, out, ws2)
    assert da.da_read_device_error(ws2) == da.DEV_ERR_LEN_RANGE
    assert torch.equal(out[0].cpu(), torch.zeros(4, 128))   # lens 16 > max_len 8
    # expected cache built on the CPU: sequence 1 received the zero row at row 5
    c["k_cache"][1, :, 5] = 0
    c["v_cache"][1, :, 5] = 0
    ref = oracle_out(w, c, lens=torch.tensor([16, 6], dtype=torch.int32))
    check_close(out[1:], ref[1:], "bf16")


# ------------------------------------------------------------------ full-size workloads
FULL = ["mha_bf16", "gqa8_bf16", "mqa_bf16", "gqa8_fp8", "gqa8_int8"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(name):
    """The workloads at their real sizes in the default launch plan; the oracle checks every
    head of every sequence."""
    w = workloads.WORKLOADS[name]
    log(f"case full {name}: generating")
    c = workloads.generate(w)
    log(f"case full {name}: running GPU, plan {da.da_plan(desc_of(w), int(c['lens_final'].max()))}")
    out, _, _, err = run_gpu(w, c)
    assert err == 0
    out = out.cpu()
    assert torch.isfinite(out).all()
    log(f"case full {name}: oracle over all {w.B} sequences")
    check_close(out, oracle_out(w, c), w.kv_dtype, name)


@pytest.mark.parametrize("form", ["one call", "two stages"])
def test_full_size_fused_decode_step(form):
    """The step the benchmark times, at full size: decode_attn_append_run on the GQA 32q/8kv
    bf16 workload (16 ragged sequences up to 32768 rows, one appended row each), in the
    one-call form and in the two-stage form the benchmark brackets with events. Every head of
    every sequence against the oracle over the oracle's own appended cache; the whole cache
    buffers bit-exact against that cache; every length one longer."""
    w = workloads.WORKLOADS["gqa8_bf16"]
    log(f"case full fused step ({form}): generating")
    c = workloads.generate(w)
    desc = desc_of(w)
    g = to_gpu(c)
    lens = g["lens_init"].clone()
    ml = int(c["lens_final"].max())
    ws = da.Workspace(desc, ml)
    out = torch.empty(w.B, w.h_q, w.d, device="cuda")
    kn, vn = g["k_new"][0].contiguous(), g["v_new"][0].contiguous()
    log(f"case full fused step ({form}): running GPU, plan {da.da_plan(desc, ml)}")
    if form == "one call":
        da.decode_attn_append_run(desc, g["q"], g["k_cache"], g["v_cache"], lens, kn, vn, ml, None, out, ws)
    else:
        da.decode_attn_append_partial(desc, g["q"], g["k_cache"], g["v_cache"], lens, kn, vn, ml, None, ws)
        da.decode_attn_append_combine(desc, lens, ml, out, ws)
    assert da.da_read_device_error(ws) == 0
    assert torch.equal(lens.cpu(), c["lens_final"])
    log(f"case full fused step ({form}): oracle append and attention")
    kc, vc = oracle._np(c["k_cache"]).copy(), oracle._np(c["v_cache"]).copy()
    ln = c["lens_init"].numpy().copy()
    oracle.kv_append(kc, vc, ln, oracle._np(c["k_new"][0]).copy(), oracle._np(c["v_new"][0]).copy())
    assert np.array_equal(oracle._np(g["k_cache"].cpu()), kc)
    assert np.array_equal(oracle._np(g["v_cache"].cpu()), vc)
    check_close(out, oracle.decode_f64(c["q"], kc, vc, ln, w.scale), "bf16", f"fused step, {form}")


def test_stream_read_reads_every_byte_once():
    """da_stream_read (the measured-ceiling helper): workgroup w folds the 32-bit words of its
    chunk by XOR; every byte of the buffer lands in exactly one workgroup's value."""
    n = (3 << 20) + 4096  # not a multiple of the per-workgroup chunk
    g = torch.Generator().manual_seed(11)
    host = torch.randint(0, 256, (n,), generator=g, dtype=torch.int32).to(torch.uint8)
    sink = torch.full((512,), -1.0, device="cuda")
    da.da_stream_read(host.cuda(), sink)
    torch.cuda.synchronize()
    step = 256 * 16 * 8
    chunk = -(-(n // 512) // step) * step
    words = host.numpy().view(np.uint32)
    expect = []
    for w in range(512):
        part = words[w * chunk // 4:min((w + 1) * chunk, n) // 4]
        expect.append(float(np.bitwise_xor.reduce(part)) if part.size else 0.0)
    assert np.array_equal(sink.cpu().numpy(), np.array(expect, dtype=np.float32))


def test_largest_batch_and_short_sequences():
    """The largest batch one call takes (1024 sequences, the prefix over lengths spread over
    every thread of the workgroup), with ragged lengths from 1 row up, on both flavours."""
    for h_q in (8, 2):  # g = 4: matrix cores; g = 1: vector ALUs
        w = W(B=1024, h_q=h_q, h_kv=2, d=64, cap=96, lens=("uniform", 1, 96), seed=90 + h_q)
        c = workloads.generate(w)
        log(f"case batch 1024 h_q={h_q}")
        out, _, _, err = run_gpu(w, c)
        assert err == 0
        check_close(out, oracle_out(w, c), "bf16", f"B=1024 h_q={h_q}")
