"""decode_attn_run_static (the entry point that allocates nothing: its partials live in the
library's static per-device scratch) against decode_attn_run with a caller workspace.

Both run the same kernels on the same partition, so their outputs must be equal bit for bit;
each is also held to the oracle's tolerance. Two calls in a row, the second on a smaller
input, show that the scratch left by one call does not leak into the next.
"""
import pytest
import torch

import decode_attention_kv_split_amd as da
import workloads
from tests.gpu_case import check_close, desc_of, log, oracle_out, to_gpu

pytestmark = pytest.mark.gpu


def _case(**kw):
    base = dict(name="static", B=4, h_q=16, h_kv=4, d=128, cap=3000, q_dtype="bf16", kv_dtype="bf16",
                lens=("uniform", 1, 3000), steps=0, seed=201, scale=workloads._inv_sqrt(128))
    base.update(kw)
    if base["kv_dtype"] == "f32":
        base["q_dtype"] = "f32"
    base["scale"] = workloads._inv_sqrt(base["d"])
    return workloads.Workload(**base)


def _both(w, lens=None):
    """(decode_attn_run output, decode_attn_run_static output, its error word) on w's inputs."""
    c = workloads.generate(w)
    g = to_gpu(c)
    lens = g["lens_final"] if lens is None else lens.cuda()
    ml = int(c["lens_final"].max())
    desc = desc_of(w)
    ws = da.Workspace(desc, ml)
    ref = torch.full(desc.rows_shape(), 5.0, device="cuda")
    da.decode_attn_run(desc, g["q"], g["k_cache"], g["v_cache"], lens, ml, g["kv_scales"], ref, ws)
    ws_err = da.da_read_device_error(ws)
    out = torch.full(desc.rows_shape(), -5.0, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    da.decode_attn_run_static(desc, g["q"], g["k_cache"], g["v_cache"], lens, ml, g["kv_scales"], out, err)
    torch.cuda.synchronize()
    return c, ref, ws_err, out, int(err.item())


def test_static_scratch_matches_workspace_run_then_a_smaller_call():
    # first call: 4 ragged sequences, g = 4 (matrix cores), many segments per unit
    w1 = _case()
    log(f"case static call 1: B={w1.B} h_q={w1.h_q} h_kv={w1.h_kv} {w1.kv_dtype}")
    c1, ref1, e1, out1, s1 = _both(w1)
    assert e1 == 0 and s1 == 0
    assert torch.equal(out1, ref1)
    check_close(out1, oracle_out(w1, c1), "bf16", "static call 1")
    # second call, smaller: 2 shorter sequences, fp8 with g = 2 (vector ALUs)
    w2 = _case(B=2, h_q=4, h_kv=2, cap=700, kv_dtype="fp8", lens=("uniform", 1, 700), seed=202)
    log(f"case static call 2: B={w2.B} h_q={w2.h_q} h_kv={w2.h_kv} {w2.kv_dtype}")
    c2, ref2, e2, out2, s2 = _both(w2)
    assert e2 == 0 and s2 == 0
    assert torch.equal(out2, ref2)
    check_close(out2, oracle_out(w2, c2), "fp8", "static call 2")


def test_static_scratch_flags_device_errors_like_the_workspace():
    """A length past max_len: zeros and DA_DEV_ERR_LEN_RANGE in the caller's error word, the
    rest equal to decode_attn_run."""
    w = _case(B=3, h_q=8, h_kv=2, cap=600, lens=("const", 600), seed=203)
    lens = torch.tensor([300, 0, 450], dtype=torch.int32)
    log("case static device error")
    c, ref, e, out, s = _both(w, lens)
    assert e == da.DEV_ERR_LEN_RANGE and s == da.DEV_ERR_LEN_RANGE
    assert torch.equal(out, ref)
    assert torch.equal(out[1].cpu(), torch.zeros(8, 128))
    ok = torch.tensor([300, 1, 450], dtype=torch.int32)
    check_close(out[[0, 2]], oracle_out(w, c, lens=ok)[[0, 2]], "bf16")


def test_static_scratch_without_error_word():
    """dev_err may be NULL: the same output, the bits dropped."""
    w = _case(B=2, h_q=32, h_kv=1, cap=2500, lens=("uniform", 2000, 2500), seed=204)
    c = workloads.generate(w)
    g = to_gpu(c)
    desc = desc_of(w)
    ml = int(c["lens_final"].max())
    log("case static without error word")
    ws = da.Workspace(desc, ml)
    ref = torch.empty(desc.rows_shape(), device="cuda")
    da.decode_attn_run(desc, g["q"], g["k_cache"], g["v_cache"], g["lens_final"], ml, None, ref, ws)
    out = torch.empty_like(ref)
    da.decode_attn_run_static(desc, g["q"], g["k_cache"], g["v_cache"], g["lens_final"], ml, None, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    check_close(out, oracle_out(w, c), "bf16")


def test_static_scratch_across_descriptors_and_paths():
    """Calls with other descriptors and both launch paths in turn on the one static scratch (the
    single pass keeps its counters in a part of the scratch nothing else writes): each equals
    decode_attn_run on a fresh workspace."""
    cases = [
        _case(B=1, h_q=1, h_kv=1, d=64, cap=1024, kv_dtype="f32", lens=("const", 1024), seed=210),   # single
        _case(B=3, h_q=32, h_kv=8, cap=2000, lens=("uniform", 1000, 2000), seed=211),               # split
        _case(B=5, h_q=8, h_kv=2, d=64, cap=300, lens=("uniform", 1, 300), seed=212),                # single
        _case(B=2, h_q=4, h_kv=4, cap=4000, kv_dtype="int8", lens=("uniform", 3000, 4000), seed=213), # split
        _case(B=1, h_q=1, h_kv=1, d=64, cap=1024, kv_dtype="f32", lens=("const", 1000), seed=214),   # single
    ]
    for rep in range(2):
        for w in cases:
            log(f"case static round {rep}: B={w.B} h_q={w.h_q} h_kv={w.h_kv} d={w.d} {w.kv_dtype} "
                f"path {da.da_plan(desc_of(w), w.cap)['path']}")
            c, ref, e, out, s = _both(w)
            assert e == 0 and s == 0
            assert torch.equal(out, ref)
            check_close(out, oracle_out(w, c), w.kv_dtype, "static across descriptors")
