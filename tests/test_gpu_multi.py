"""Multi-query causal decode on the GPU (descriptor n_queries = T > 1) against the oracle.

Query t of sequence b attends over rows [0, lens[b] - T + 1 + t). The cases cover every
kernel flavour (matrix cores with head tiles of 3 to 32 query rows in 16 or 32 slots, bf16
through the register ring, fp8 / int8 through the LDS stages; the vector ALUs for fp32 and for
groups of at most 2 query rows), lengths equal to T (the first query sees one row), workgroup
shares small enough that whole segments lie past some queries' causal bound, and invalid
lengths (lens < T).
"""
import numpy as np
import pytest
import torch

import decode_attention_kv_split_amd as da
import oracle
import workloads
from tests.gpu_case import check_close, log, to_gpu

pytestmark = pytest.mark.gpu


def mq_workload(kv, d, h_q, h_kv, T, lens, cap, seed):
    return workloads.Workload("mq", 5, h_q, h_kv, d, cap, "f32" if kv == "f32" else "bf16", kv, lens, 0, seed,
                              workloads._inv_sqrt(d), nq=T)


def run_multi(w, c, block_rows=0, max_len=None, path=da.PATH_AUTO):
    desc = da.Desc(w.B, w.h_q, w.h_kv, w.d, w.cap, workloads.TORCH_DTYPE[w.q_dtype],
                   workloads.TORCH_DTYPE[w.kv_dtype], w.scale, block_rows, w.nq, da.FLAVOUR_AUTO, path)
    g = to_gpu(c)
    ml = max_len or int(c["lens_final"].max())
    ws = da.Workspace(desc, ml)
    out = torch.full(desc.rows_shape(), 7.0, device="cuda")
    da.decode_attn_run(desc, g["q"], g["k_cache"], g["v_cache"], g["lens_final"], ml, g["kv_scales"], out, ws)
    return out, da.da_read_device_error(ws)


CASES = [
    # kv, d, h_q, h_kv, T, block_rows
    ("bf16", 128, 32, 8, 4, 0),      # g*T = 16: matrix cores, one 16-row tile per KV head
    ("bf16", 128, 8, 8, 4, 256),     # MHA with 4 queries: g*T = 4 on the matrix cores
    ("bf16", 128, 8, 8, 3, 0),       # g*T = 3: matrix cores, 3 rows in 16 slots
    ("bf16", 64, 16, 2, 2, 37),      # d = 64, many small segments
    ("bf16", 128, 32, 1, 8, 0),      # MQA with 8 queries: g*T = 256, 32-row tiles
    ("f32", 64, 4, 2, 3, 100),       # fp32: vector ALUs, 6 rows in 8 slots
    ("fp8", 128, 16, 2, 4, 0),       # fp8, LDS stages, 32-row tiles (two head tiles)
    ("int8", 128, 8, 1, 2, 37),      # int8, LDS stages, 16-row tiles, many segments
    ("int8", 64, 12, 4, 5, 0),       # int8 d = 64, g*T = 15: one 16-slot tile
    ("bf16", 128, 8, 8, 2, 100),     # g*T = 2: vector ALUs, one tile
    ("bf16", 64, 20, 4, 4, 0),       # g*T = 20: one 32-slot tile
    ("fp8", 128, 14, 2, 4, 300),     # g*T = 28: one 32-slot tile
    ("f32", 128, 8, 1, 3, 0),        # fp32, g*T = 24: three 8-row tiles
    ("bf16", 128, 8, 2, 64, 0),      # a 64-row prefill chunk: g*T = 256, eight 32-row tiles per KV head
    ("fp8", 128, 4, 4, 40, 500),     # fp8 chunk of 40 rows, MHA: g*T = 40 -> two 20-row tiles
]


@pytest.mark.parametrize("path", [da.PATH_SPLIT, da.PATH_SINGLE])
@pytest.mark.parametrize("kv,d,h_q,h_kv,T,block_rows", CASES)
def test_multi_query_parity(kv, d, h_q, h_kv, T, block_rows, path):
    seed = 500 + CASES.index((kv, d, h_q, h_kv, T, block_rows))
    w = mq_workload(kv, d, h_q, h_kv, T, ("uniform", T, 1500), 1500, seed)
    c = workloads.generate(w)
    c["lens_final"][0] = T  # the first query of sequence 0 sees exactly one row
    log(f"case multi {kv} d={d} h_q={h_q} h_kv={h_kv} T={T} block_rows={block_rows} path={path} "
        f"lens={c['lens_final'].tolist()}")
    out, err = run_multi(w, c, block_rows if path == da.PATH_SPLIT else 0, path=path)
    assert err == 0
    ref = oracle.decode_multi_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale,
                                  kv_scales=c["kv_scales"])
    check_close(out, ref, kv, "multi-query")


def test_single_query_descriptor_is_the_decode_path():
    """n_queries = 1 and the default (0) run the single-query decode: identical bits."""
    w = workloads.Workload("mq1", 4, 16, 4, 128, 900, "bf16", "bf16", ("uniform", 1, 900), 0, 41,
                           workloads._inv_sqrt(128))
    c = to_gpu(workloads.generate(w))
    outs = []
    for nq in (0, 1):
        desc = da.Desc(w.B, w.h_q, w.h_kv, w.d, w.cap, torch.bfloat16, torch.bfloat16, w.scale, 0, nq)
        ws = da.Workspace(desc, 900)
        out = torch.empty(w.B, w.h_q, w.d, device="cuda")
        da.decode_attn_run(desc, c["q"], c["k_cache"], c["v_cache"], c["lens_final"], 900, None, out, ws)
        outs.append(out.cpu())
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("path", [da.PATH_SPLIT, da.PATH_SINGLE])
def test_lengths_shorter_than_T_are_flagged(path):
    """A sequence with fewer rows than query rows has no causal prefix for its first queries:
    its output is zeroed and DA_DEV_ERR_LEN_RANGE raised; the other sequences are unaffected."""
    T = 4
    w = mq_workload("bf16", 128, 8, 2, T, ("uniform", T, 600), 600, 77)
    c = workloads.generate(w)
    lens = c["lens_final"].clone()
    lens[2] = T - 1
    c2 = dict(c, lens_final=lens)
    out, err = run_multi(w, c2, 0, 600, path)
    assert err == da.DEV_ERR_LEN_RANGE
    o = out.cpu()
    assert torch.equal(o[2], torch.zeros_like(o[2]))
    keep = [0, 1, 3, 4]
    ref = oracle.decode_multi_f64(c["q"][keep], c["k_cache"][keep], c["v_cache"][keep], lens[keep], w.scale)
    check_close(o[keep], ref, "bf16", "neighbours of the short sequence")


def test_multi_query_runs_are_deterministic():
    w = mq_workload("bf16", 128, 32, 8, 4, ("uniform", 4, 2000), 2000, 78)
    c = workloads.generate(w)
    a, _ = run_multi(w, c)
    b, _ = run_multi(w, c)
    assert torch.equal(a, b)


def test_full_size_multi_query_workload():
    """The 4-query GQA workload at its real size in the default plan; the oracle checks every
    (query, head) of every sequence."""
    w = workloads.WORKLOADS["gqa8_mq4_bf16"]
    log("case full gqa8_mq4_bf16: generating")
    c = workloads.generate(w)
    out, err = run_multi(w, c)
    assert err == 0
    out = out.cpu()
    assert torch.isfinite(out).all()
    log(f"case full gqa8_mq4_bf16: oracle over all {w.B} sequences")
    ref = oracle.decode_multi_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale)
    check_close(out, ref, "bf16", "full multi-query")
