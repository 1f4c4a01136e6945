"""Parity of the shard entry points on the GPU, through the C ABI, with the CPU oracle:
decode_attn_run_lse (attention over one part of every sequence's rows, with each query row's
log-sum-exp) and decode_attn_merge_lse (the log-sum-exp merge of parts), which together are
what one device runs when a context is split over several (each holds a contiguous part of
every sequence's rows and, after an all-gather of the parts' results, merges them). Head
sharding needs no new entry point: every device runs decode_attn_run on its KV heads, and the
outputs concatenate on the head axis (checked here too). Twenty-four seeded random splits
(cache type, head size, group, batch, lengths, parts and cut points, partition) close the
file.

Tolerances: out as the other parity tests (tests/gpu_case.py: the cache type's contract and
the regression bound); lse (natural log, magnitude ln n + the largest score, at most about 20
here) within LSE_ABS = 1e-5 absolute of the fp64 oracle. Parts are NaN-poisoned past their lengths, as
the workloads' caches are, so that a read out of range shows up as a non-finite output.
"""
import dataclasses

import numpy as np
import pytest
import torch

import decode_attention_kv_split_amd as da
import oracle
import workloads
from tests.gpu_case import check_close, desc_of, log, to_gpu

pytestmark = pytest.mark.gpu

# fp32 log-sum-exp: the merged sum of exponentials and the scores carry a few ulp of relative
# error each. The bound is about eight times the largest error measured over these tests on the
# GPU (1.3e-6); a mistake in the formula (a missing maximum or ln 2, the maximum of one wave
# instead of the merged one) moves lse by O(1).
LSE_ABS = 1e-5


def W(**kw):
    base = dict(name="shard", B=4, h_q=8, h_kv=2, d=128, cap=3000, q_dtype="bf16", kv_dtype="bf16",
                lens=("uniform", 1, 3000), steps=0, seed=5, scale=workloads._inv_sqrt(128))
    base.update(kw)
    if base["kv_dtype"] == "f32":
        base["q_dtype"] = "f32"
    base["scale"] = workloads._inv_sqrt(base["d"])
    return workloads.Workload(**base)


def _desc(w, cap=None):
    return dataclasses.replace(desc_of(w), cap=w.cap if cap is None else cap, n_queries=w.nq)


def check_lse(got: torch.Tensor, ref: np.ndarray, what: str) -> float:
    g = got.detach().cpu().double().numpy()
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.array_equal(np.isneginf(g), np.isneginf(ref)), f"{what}: -inf rows differ"
    fin = np.isfinite(ref)
    assert np.isfinite(g[fin]).all(), f"{what}: non-finite lse"
    err = float(np.abs(g[fin] - ref[fin]).max()) if fin.any() else 0.0
    log(f"  {what}: lse max abs error {err:.2e}")
    assert err <= LSE_ABS, f"{what}: lse error {err:.3e} exceeds {LSE_ABS:.0e}"
    return err


def run_lse(w, desc, q, kc, vc, lens, max_len, scales):
    out = torch.empty(desc.rows_shape(), dtype=torch.float32, device="cuda")
    lse = torch.empty(desc.rows_shape()[:-1], dtype=torch.float32, device="cuda")
    ws = da.Workspace(desc, max_len)
    da.decode_attn_run_lse(desc, q, kc, vc, lens, max_len, scales, out, lse, ws)
    assert da.da_read_device_error(ws) == 0
    return out, lse


# (kv, d, h_q, h_kv, T, B, lens): every flavour (vector ALUs, the 16- and 32-slot register
# rings, the LDS stages), several query rows, and a batch beyond 64 sequences (the walk's
# prefix in LDS)
CASES = [
    ("bf16", 128, 8, 2, 1, 4, ("uniform", 1, 3000)),
    ("bf16", 128, 32, 1, 1, 2, ("uniform", 1, 5000)),
    ("bf16", 64, 4, 4, 1, 3, ("uniform", 1, 2000)),
    ("f32", 64, 4, 1, 1, 3, ("uniform", 1, 2500)),
    ("fp8", 128, 16, 2, 1, 3, ("uniform", 1, 3000)),
    ("int8", 128, 8, 1, 1, 3, ("uniform", 1, 3000)),
    ("bf16", 128, 8, 2, 4, 3, ("uniform", 4, 2000)),
    ("bf16", 128, 8, 2, 1, 80, ("uniform", 1, 300)),
]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_run_lse_against_oracle_and_two_stage_form(i):
    """out and lse against the oracle, with one or two sequences empty (lens 0: out 0, lse -inf, no
    device error); out bit for bit equal to decode_attn_partial + decode_attn_combine, which
    run the same two kernels."""
    kv, d, h_q, h_kv, T, B, lens = CASES[i]
    w = W(kv_dtype=kv, d=d, h_q=h_q, h_kv=h_kv, nq=T, B=B, lens=lens, cap=lens[2], seed=100 + i)
    c = workloads.generate(w)
    lens_t = c["lens_final"].clone()
    lens_t[0] = 0
    if B > 2:
        lens_t[B - 1] = 0
    log(f"case run_lse kv={kv} d={d} h_q={h_q} h_kv={h_kv} T={T} B={B}")
    desc = _desc(w)
    g = to_gpu(c)
    ml = int(c["lens_final"].max())
    ln = lens_t.to("cuda")
    out, lse = run_lse(w, desc, g["q"], g["k_cache"], g["v_cache"], ln, ml, g["kv_scales"])
    ref_o, ref_l = oracle.decode_lse_f64(c["q"], c["k_cache"], c["v_cache"], lens_t, w.scale, kv_scales=c["kv_scales"])
    live = lens_t > 0
    check_close(out[live.to("cuda")], ref_o[live.numpy()], kv, "run_lse out")
    assert torch.count_nonzero(out[~live.to("cuda")]) == 0
    check_lse(lse, ref_l, "run_lse lse")
    # the two-stage form on the live sequences only (it flags an empty sequence)
    sub = live.nonzero().flatten()
    wl = w.resized(B=len(sub))
    dl = _desc(wl)
    q2 = g["q"][sub.to("cuda")].contiguous()
    k2, v2 = g["k_cache"][sub.to("cuda")].contiguous(), g["v_cache"][sub.to("cuda")].contiguous()
    s2 = None if g["kv_scales"] is None else g["kv_scales"][sub.to("cuda")].contiguous()
    l2 = lens_t[sub].to("cuda")
    o2 = torch.empty(dl.rows_shape(), dtype=torch.float32, device="cuda")
    lse2 = torch.empty(dl.rows_shape()[:-1], dtype=torch.float32, device="cuda")
    ws2 = da.Workspace(dl, ml)
    da.decode_attn_run_lse(dl, q2, k2, v2, l2, ml, s2, o2, lse2, ws2)
    o3 = torch.empty_like(o2)
    da.decode_attn_partial(dl, q2, k2, v2, l2, ml, s2, ws2)
    da.decode_attn_combine(dl, l2, ml, o3, ws2)
    assert da.da_read_device_error(ws2) == 0
    assert torch.equal(o2, o3)


def split_rows(c, cuts, kv):
    """Part p of the caches: rows [cuts[b][p], cuts[b][p+1]) of sequence b as a cache of its own
    (NaN-poisoned past its length), with its lengths."""
    k, v = c["k_cache"], c["v_cache"]
    B, h_kv, cap, d = k.shape
    parts = []
    for p in range(len(cuts[0]) - 1):
        lens = torch.tensor([cuts[b][p + 1] - cuts[b][p] for b in range(B)], dtype=torch.int32)
        cp = max(1, int(lens.max()))
        kp, vp = workloads._poisoned((B, h_kv, cp, d), kv), workloads._poisoned((B, h_kv, cp, d), kv)
        for b in range(B):
            n = int(lens[b])
            kp[b, :, :n] = k[b, :, cuts[b][p]:cuts[b][p] + n]
            vp[b, :, :n] = v[b, :, cuts[b][p]:cuts[b][p] + n]
        parts.append((kp, vp, lens))
    return parts


@pytest.mark.parametrize("kv,h_q,h_kv,P,seed", [
    ("bf16", 32, 1, 2, 0), ("bf16", 32, 1, 8, 1), ("bf16", 8, 2, 3, 2), ("fp8", 16, 2, 4, 3),
    ("int8", 8, 1, 5, 4), ("f32", 4, 1, 3, 5)])
def test_context_split_then_merge_equals_attention_over_all_rows(kv, h_q, h_kv, P, seed):
    """Cut every sequence's rows into P contiguous parts at random places (empty parts
    included), run decode_attn_run_lse on each part as its own cache, merge the P results with
    decode_attn_merge_lse: the result is the attention over all the rows (oracle), and the
    merge kernel equals the oracle's merge of the same GPU part results."""
    d = 64 if kv == "f32" else 128
    w = W(kv_dtype=kv, d=d, h_q=h_q, h_kv=h_kv, B=4, cap=6000, lens=("uniform", 1, 6000), seed=40 + seed)
    c = workloads.generate(w)
    rng = np.random.default_rng(seed)
    cuts = [[0] + sorted(int(x) for x in rng.integers(0, n + 1, P - 1)) + [n] for n in c["lens_final"].tolist()]
    log(f"case context split kv={kv} h_q={h_q} h_kv={h_kv} P={P} lens={c['lens_final'].tolist()}")
    q = c["q"].to("cuda")
    sc = None if c["kv_scales"] is None else c["kv_scales"].to("cuda")
    outs, lses = [], []
    for kp, vp, lp in split_rows(c, cuts, kv):
        ml = max(1, int(lp.max()))
        desc = _desc(w, cap=kp.shape[2])
        o, l = run_lse(w, desc, q, kp.to("cuda"), vp.to("cuda"), lp.to("cuda"), ml, sc)
        outs.append(o)
        lses.append(l)
    outs, lses = torch.stack(outs), torch.stack(lses)
    out = torch.empty(w.B, w.h_q, w.d, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.B, w.h_q, dtype=torch.float32, device="cuda")
    da.decode_attn_merge_lse(outs, lses, out, lse)
    ref_o, ref_l = oracle.decode_lse_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale,
                                         kv_scales=c["kv_scales"])
    check_close(out, ref_o, kv, "merged out")
    check_lse(lse, ref_l, "merged lse")
    # the merge kernel alone, on the GPU's own part results
    mo, ml_ = oracle.merge_lse(outs.cpu().double().numpy(), lses.cpu().double().numpy())
    np.testing.assert_allclose(out.cpu().double().numpy(), mo, rtol=0, atol=1e-5 * max(1.0, float(np.abs(mo).max())))
    check_lse(lse, ml_, "merge kernel lse")


@pytest.mark.parametrize("d", [64, 128, 4, 12])
def test_merge_kernel_edge_cases(d):
    """One part: unchanged, bit for bit. A part with lse -inf (no rows) weighs nothing; a row
    no part holds gets out 0 and lse -inf; a part 800 below the others weighs nothing (no
    NaN); lse is optional. Row counts that are not multiples of the workgroup."""
    gen = torch.Generator().manual_seed(d)
    for rows in (1, 37, 1000):
        o = torch.randn(3, rows, d, generator=gen)
        l = torch.randn(3, rows, generator=gen) * 5
        l[1, : rows // 2] = -float("inf")
        l[:, rows - 1] = -float("inf")
        l[2, rows // 3] -= 800
        og, lg = o.cuda(), l.cuda()
        out = torch.empty(rows, d, device="cuda")
        lse = torch.empty(rows, device="cuda")
        da.decode_attn_merge_lse(og[:1].contiguous(), lg[:1].contiguous(), out, lse)
        fin = torch.isfinite(l[0])
        assert torch.equal(out.cpu()[fin], o[0][fin]) and torch.equal(lse.cpu(), l[0])
        assert torch.count_nonzero(out.cpu()[~fin]) == 0
        da.decode_attn_merge_lse(og, lg, out, lse)
        ref_o, ref_l = oracle.merge_lse(o.double().numpy(), l.double().numpy())
        got = out.cpu().double().numpy()
        assert np.isfinite(got).all()
        np.testing.assert_allclose(got, ref_o, rtol=0, atol=1e-5)
        check_lse(lse, ref_l, f"merge d={d} rows={rows}")
        out2 = torch.empty_like(out)
        da.decode_attn_merge_lse(og, lg, out2, None)
        assert torch.equal(out, out2)


def test_full_size_mqa_context_share():
    """The long-context MQA workload (4 sequences of 131072 rows, 32 query heads, bf16) split
    into 8 parts of 16384 rows, one device's share each: the 8 part results merged equal the
    oracle over all the rows (every head of two sequences) and decode_attn_run over the whole
    cache."""
    w = workloads.WORKLOADS["mqa_bf16"]
    c = workloads.generate(w)
    P = 8
    n = int(c["lens_final"][0])
    assert all(int(x) == n for x in c["lens_final"]) and n % P == 0
    log(f"case full-size MQA share: B={w.B} n={n} P={P}")
    g = to_gpu(c)
    part = n // P
    desc = _desc(w, cap=part)
    outs, lses = [], []
    for p in range(P):
        kp = g["k_cache"][:, :, p * part:(p + 1) * part].contiguous()
        vp = g["v_cache"][:, :, p * part:(p + 1) * part].contiguous()
        lp = torch.full((w.B,), part, dtype=torch.int32, device="cuda")
        o, l = run_lse(w, desc, g["q"], kp, vp, lp, part, None)
        outs.append(o)
        lses.append(l)
    out = torch.empty(w.B, w.h_q, w.d, device="cuda")
    lse = torch.empty(w.B, w.h_q, device="cuda")
    da.decode_attn_merge_lse(torch.stack(outs), torch.stack(lses), out, lse)
    whole = torch.empty_like(out)
    dw = desc_of(w)
    ws = da.Workspace(dw, n)
    da.decode_attn_run(dw, g["q"], g["k_cache"], g["v_cache"], g["lens_final"], n, None, whole, ws)
    assert da.da_read_device_error(ws) == 0
    for b in (0, w.B - 1):
        sl = slice(b, b + 1)
        ref_o, ref_l = oracle.decode_lse_f64(c["q"][sl].contiguous(), c["k_cache"][sl].contiguous(),
                                             c["v_cache"][sl].contiguous(), c["lens_final"][sl], w.scale)
        check_close(out[sl], ref_o, "bf16", f"merged MQA share b={b}")
        check_lse(lse[sl], ref_l, f"merged MQA lse b={b}")
        check_close(whole[sl], ref_o, "bf16", f"whole MQA b={b}")


def test_head_split_concat_equals_whole():
    """Head sharding: 4 devices of 2 KV heads (8 query heads) each run decode_attn_run on their
    heads; the outputs, concatenated on the head axis, are the attention of all 32 heads
    (oracle, and decode_attn_run on all heads within the tolerance)."""
    w = W(B=6, h_q=32, h_kv=8, cap=5000, lens=("uniform", 512, 5000), seed=77)
    c = workloads.generate(w)
    g = to_gpu(c)
    ml = int(c["lens_final"].max())
    P, kh = 4, w.h_kv // 4
    qh = w.h_q // P
    parts = []
    for p in range(P):
        wp = w.resized(h_q=qh, h_kv=kh)
        dp = desc_of(wp)
        o = torch.empty(w.B, qh, w.d, device="cuda")
        ws = da.Workspace(dp, ml)
        da.decode_attn_run(dp, g["q"][:, p * qh:(p + 1) * qh].contiguous(), g["k_cache"][:, p * kh:(p + 1) * kh].contiguous(),
                           g["v_cache"][:, p * kh:(p + 1) * kh].contiguous(), g["lens_final"], ml, None, o, ws)
        assert da.da_read_device_error(ws) == 0
        parts.append(o)
    out = torch.cat(parts, dim=1)
    ref = oracle.decode_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale)
    check_close(out, ref, "bf16", "head shards concatenated")
    whole = torch.empty_like(out)
    dw = desc_of(w)
    ws = da.Workspace(dw, ml)
    da.decode_attn_run(dw, g["q"], g["k_cache"], g["v_cache"], g["lens_final"], ml, None, whole, ws)
    check_close(whole, ref, "bf16", "all heads")


def draw_split_cases(n=24, seed=4242):
    """Random context splits: cache type, head size, group, batch, lengths, the number of parts
    and where each sequence is cut (empty parts included), and the partition (the library's
    own or small shares)."""
    import random
    rng = random.Random(seed)
    groups = [(1, 1), (4, 1), (8, 2), (32, 8), (32, 1), (6, 3), (12, 4), (64, 8)]
    cases = []
    for i in range(n):
        kv = rng.choice(["f32", "bf16", "bf16", "fp8", "int8"])
        d = rng.choice([64, 128])
        h_q, h_kv = rng.choice(groups)
        B = rng.randint(1, 5)
        cap = rng.choice([64, 500, 3000])
        P = rng.randint(2, 6)
        block_rows = rng.choice([0, 0, 16, 200])
        cases.append((i, kv, d, h_q, h_kv, B, cap, P, block_rows, rng.randint(0, 1 << 30)))
    return cases


SPLIT_CASES = draw_split_cases()


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[f"s{c[0]}" for c in SPLIT_CASES])
def test_random_context_split(case):
    i, kv, d, h_q, h_kv, B, cap, P, block_rows, cut_seed = case
    w = workloads.Workload("split", B, h_q, h_kv, d, cap, "f32" if kv == "f32" else "bf16", kv,
                           ("uniform", 1, cap), 0, 9000 + i, workloads._inv_sqrt(d))
    c = workloads.generate(w)
    rng = np.random.default_rng(cut_seed)
    cuts = [[0] + sorted(int(x) for x in rng.integers(0, n + 1, P - 1)) + [n] for n in c["lens_final"].tolist()]
    log(f"case random split s{i}: {kv} d={d} h_q={h_q} h_kv={h_kv} B={B} cap={cap} P={P} block_rows={block_rows} "
        f"lens={c['lens_final'].tolist()}")
    q = c["q"].to("cuda")
    sc = None if c["kv_scales"] is None else c["kv_scales"].to("cuda")
    outs, lses = [], []
    for kp, vp, lp in split_rows(c, cuts, kv):
        ml = max(1, int(lp.max()))
        desc = dataclasses.replace(desc_of(w), cap=kp.shape[2], block_rows=block_rows)
        o, l = run_lse(w, desc, q, kp.to("cuda"), vp.to("cuda"), lp.to("cuda"), ml, sc)
        outs.append(o)
        lses.append(l)
    out = torch.empty(w.B, w.h_q, w.d, device="cuda")
    lse = torch.empty(w.B, w.h_q, device="cuda")
    da.decode_attn_merge_lse(torch.stack(outs), torch.stack(lses), out, lse)
    ref_o, ref_l = oracle.decode_lse_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale,
                                         kv_scales=c["kv_scales"])
    check_close(out, ref_o, kv, f"s{i} merged out")
    check_lse(lse, ref_l, f"s{i} merged lse")
