"""Pins of the CPU oracle against things other than itself.

Each test ties the fp64 oracle to a value the pages print, a closed form, a
library routine the pages name as ground truth (PyTorch SDPA), an independent
50-digit brute force, or an invariant the pages state. None of these tests
touches the GPU or the HIP library.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import workloads



def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked example
def test_worked_example_printed_values(golden_dir):
    """Page "MoA-Structured Decode Attention", §2 concrete example, Steps I-III."""
    ex = _load(golden_dir, "moa_worked_example.json")
    q = np.array(ex["inputs"]["q"])
    K = np.array(ex["inputs"]["K"])
    V = np.array(ex["inputs"]["V"])
    scale = 1.0 / math.sqrt(ex["inputs"]["scale_inv_sqrt"])
    # the printed Step I partial products
    for l, (p0, p1) in enumerate(ex["printed_step1_partials"]):
        assert q[0] * K[l, 0] == p0 and q[1] * K[l, 1] == p1
    r = oracle.head_f64(q, K, V, scale)
    pr = ex["printed"]
    np.testing.assert_allclose(r["s"], pr["s"]["values"], rtol=0, atol=pr["s"]["abs_tol"])
    assert abs(r["m"] - pr["m"]["value"]) <= pr["m"]["abs_tol"]
    np.testing.assert_allclose(r["e"], pr["e"]["values"], rtol=0, atol=pr["e"]["abs_tol"])
    assert abs(r["Z"] - pr["Z"]["value"]) <= pr["Z"]["abs_tol"]
    np.testing.assert_allclose(r["a"], pr["a"]["values"], rtol=0, atol=pr["a"]["abs_tol"])
    np.testing.assert_allclose(r["out"], pr["out"]["values"], rtol=0, atol=pr["out"]["abs_tol"])


def test_worked_example_closed_form(golden_dir):
    """The example in closed form: e1 = exp(-1/sqrt 2), Z = 1 + e1, out = a0 V0 + a1 V1."""
    ex = _load(golden_dir, "moa_worked_example.json")
    V = np.array(ex["inputs"]["V"])
    r = oracle.head_f64(ex["inputs"]["q"], ex["inputs"]["K"], V, 1 / math.sqrt(2))
    e1 = math.exp(-1 / math.sqrt(2))
    assert r["e"][0] == 1.0
    assert abs(r["e"][1] - e1) < 1e-16
    assert abs(r["Z"] - (1 + e1)) < 1e-15
    a0, a1 = 1 / (1 + e1), e1 / (1 + e1)
    np.testing.assert_allclose(r["out"], [a0 * 2 + a1 * 6, a0 * 4 + a1 * 8], rtol=0, atol=1e-14)


# ---------------------------------------------------------------- brute force
def _widen(x: torch.Tensor, scales=None, which=None) -> np.ndarray:
    """Widen typed tensors with torch's own casts (independent of the oracle's decoders)."""
    v = x.to(torch.float64)
    if scales is not None:
        v = v * scales[..., which].to(torch.float64)[..., None, None]
    return v.numpy()


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8", "int8"])
def test_oracle_vs_decimal_brute_force(seed, kv):
    """Tiny random cases (GQA, ragged n <= 8, d <= 4) against 50-digit arithmetic."""
    rng = np.random.default_rng(100 * seed + len(kv))
    h_kv = int(rng.integers(1, 3))
    g = int(rng.integers(1, 3))
    B, d, cap = 2, int(rng.integers(1, 5)), 8
    w = workloads.Workload("tiny", B, h_kv * g, h_kv, d, cap, "bf16" if kv in workloads.SCALED else kv, kv,
                           ("uniform", 1, cap), 0, 1000 + seed, 0.5 + seed / 7)
    c = workloads.generate(w, poison=False)
    got = oracle.decode_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale,
                            kv_scales=c["kv_scales"])
    sc = c["kv_scales"]
    K = _widen(c["k_cache"], sc, 0)
    V = _widen(c["v_cache"], sc, 1)
    ref = brute.decode(_widen(c["q"]).tolist(), K.tolist(), V.tolist(),
                       c["lens_final"].tolist(), float(np.float32(w.scale)))
    np.testing.assert_allclose(got, np.array(ref, dtype=np.float64), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- SDPA (the page's ground truth)
@pytest.mark.parametrize("name,h_q,h_kv,d,kv", [
    ("mha", 4, 4, 64, "bf16"), ("gqa4", 8, 2, 128, "bf16"), ("mqa", 8, 1, 64, "f32"),
    ("fp8", 8, 2, 128, "fp8"), ("int8", 8, 1, 128, "int8")])
def test_oracle_vs_torch_sdpa_fp64(name, h_q, h_kv, d, kv):
    """torch SDPA in fp64 on the CPU, per sequence, with (B, H, S, D) wrapping and
    GQA by repeat_interleave (page "MoA-Structured Decode Attention", SDPA as ground truth)."""
    w = workloads.Workload(name, 3, h_q, h_kv, d, 700, "f32" if kv == "f32" else "bf16", kv,
                           ("uniform", 1, 700), 0, 7, 1 / math.sqrt(d))
    c = workloads.generate(w, poison=True)
    got = oracle.decode_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale,
                            kv_scales=c["kv_scales"])
    sc = c["kv_scales"]
    K = torch.from_numpy(_widen(c["k_cache"], sc, 0))
    V = torch.from_numpy(_widen(c["v_cache"], sc, 1))
    q = c["q"].to(torch.float64)
    for b in range(w.B):
        n = int(c["lens_final"][b])
        kb = K[b, :, :n].repeat_interleave(w.g, dim=0)[None]
        vb = V[b, :, :n].repeat_interleave(w.g, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[b][None, :, None, :], kb, vb, scale=float(np.float32(w.scale)))
        np.testing.assert_allclose(got[b], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- invariants
def _rand_case(seed, B=2, h_q=4, h_kv=2, d=16, cap=40, kv="f32"):
    w = workloads.Workload("inv", B, h_q, h_kv, d, cap, "f32" if kv == "f32" else "bf16", kv,
                           ("uniform", 1, cap), 0, seed, 0.25)
    return w, workloads.generate(w, poison=False)


def test_convex_combination_bounds():
    """I1: softmax weights are >= 0 and sum to 1, so out lies in the per-column hull of V rows."""
    w, c = _rand_case(11)
    out = oracle.decode_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale)
    V = c["v_cache"].double().numpy()
    for b in range(w.B):
        n = int(c["lens_final"][b])
        for h in range(w.h_q):
            rows = V[b, h // w.g, :n]
            assert np.all(out[b, h] >= rows.min(0) - 1e-12)
            assert np.all(out[b, h] <= rows.max(0) + 1e-12)


def test_special_cases_reduce_to_rows_or_mean():
    """I1 special cases: n = 1 gives V[0]; equal V rows give that row; q = 0 gives the mean;
    one dominant score gives its row."""
    rng = np.random.default_rng(5)
    d, n = 8, 12
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    q = rng.standard_normal(d)
    assert np.array_equal(oracle.head_f64(q, K[:1], V[:1], 0.3)["out"], V[0])
    Veq = np.tile(V[3], (n, 1))
    np.testing.assert_allclose(oracle.head_f64(q, K, Veq, 0.3)["out"], V[3], rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.head_f64(np.zeros(d), K, V, 0.3)["out"], V.mean(0),
                               rtol=0, atol=1e-14)
    # row 7 aligned with q and scaled so its score exceeds every other by >= 40
    Kd = K.copy()
    Kd[7] = q / np.linalg.norm(q) * 200.0
    r = oracle.head_f64(q, Kd, V, 1.0)
    assert r["s"][7] - np.delete(r["s"], 7).max() >= 40
    np.testing.assert_allclose(r["out"], V[7], rtol=0, atol=1e-15)


def test_softmax_shift_cancels():
    """Step II: subtracting m does not change the softmax (the m terms cancel)."""
    rng = np.random.default_rng(9)
    q, K, V = rng.standard_normal(16), rng.standard_normal((50, 16)), rng.standard_normal((50, 16))
    r = oracle.head_f64(q, K, V, 0.7)
    e = np.exp(0.7 * (K @ q))  # unshifted exponentials, |s| << 700
    np.testing.assert_allclose(r["a"], e / e.sum(), rtol=1e-14, atol=0)
    np.testing.assert_allclose(r["out"], (e / e.sum()) @ V, rtol=0, atol=1e-14)


def test_heads_concat_equals_batched():
    """I2 (page "Phase 3, Section 6: StoryLM-0 head-parallel attention", §4 and §7(b)):
    per-head calls on one-head slices, concatenated, equal the batched-head call."""
    w, c = _rand_case(13, h_q=6, h_kv=6)
    full = oracle.decode_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale)
    parts = [oracle.decode_f64(c["q"][:, h:h + 1].contiguous(), c["k_cache"][:, h:h + 1].contiguous(),
                               c["v_cache"][:, h:h + 1].contiguous(), c["lens_final"], w.scale)
             for h in range(w.h_q)]
    assert np.array_equal(np.concatenate(parts, axis=1), full)


def test_gqa_equals_mha_on_broadcast_kv():
    """I3 (page "MoA-Structured Decode Attention", §6): selecting the KV group equals MHA
    on explicitly broadcast (repeat_interleave) KV."""
    w, c = _rand_case(17, h_q=8, h_kv=2, kv="bf16")
    gqa = oracle.decode_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale)
    kb = c["k_cache"].repeat_interleave(w.g, dim=1).contiguous()
    vb = c["v_cache"].repeat_interleave(w.g, dim=1).contiguous()
    mha = oracle.decode_f64(c["q"], kb, vb, c["lens_final"], w.scale)
    assert np.array_equal(gqa, mha)


def test_append_then_attend_prefix_invariance():
    """I4 (page "MoA-Structured Decode Attention", §5; page "Phase 3, Section 6", §4 causal
    non-leak): the output after step t equals attention over the first n_t rows of the
    final cache, and appending rows never changes earlier outputs."""
    w = workloads.WORKLOADS["single_head_f32"]
    c = workloads.generate(w)
    kc = c["k_cache"].numpy().copy()
    vc = c["v_cache"].numpy().copy()
    lens = c["lens_init"].numpy().copy()
    outs = []
    for t in range(w.steps):
        oracle.kv_append(kc, vc, lens, c["k_new"][t].numpy().copy(), c["v_new"][t].numpy().copy())
        assert int(lens[0]) == 1009 + t
        outs.append(oracle.decode_f64(c["q"], kc, vc, lens, w.scale))
    final_k, final_v = kc.copy(), vc.copy()
    for t in range(w.steps):
        n_t = np.array([1009 + t], dtype=np.int32)
        assert np.array_equal(outs[t], oracle.decode_f64(c["q"], final_k, final_v, n_t, w.scale))
    # after 16 steps the cache holds all 1024 drawn rows in order
    assert not np.isnan(final_k).any() and not np.isnan(final_v).any()


def test_append_layout_gamma_offsets(golden_dir):
    """I5 (page "MoA-Structured Decode Attention", §4 gamma offsets, §5 append): appending the
    n = 3, d = 2 example row by row lays element (l, j) at flat offset l*2 + j."""
    ex = _load(golden_dir, "moa_gamma_offsets.json")
    n, d = ex["n"], ex["d"]
    kc = np.full((1, 1, n, d), -1.0, dtype=np.float32)
    vc = np.full((1, 1, n, d), -1.0, dtype=np.float32)
    lens = np.zeros(1, dtype=np.int32)
    for l in range(n):
        row = np.array([[[10 * l + j for j in range(d)]]], dtype=np.float32)
        oracle.kv_append(kc, vc, lens, row, row + 100)
    flat = kc.reshape(-1)
    for l in range(n):
        for j in range(d):
            assert flat[ex["offsets"][l][j]] == 10 * l + j
    with pytest.raises(ValueError):  # a full sequence refuses the append and is unchanged
        oracle.kv_append(kc, vc, lens, row, row)
    assert int(lens[0]) == n


def test_append_is_bit_exact_and_touches_only_its_rows():
    """I5: after appends the cache equals a host-built expected buffer bit for bit."""
    w = workloads.Workload("app", 3, 8, 4, 32, 10, "bf16", "bf16", ("uniform", 3, 10), 2, 21, 0.2)
    c = workloads.generate(w)
    kc = c["k_cache"].view(torch.int16).numpy().view(np.uint16).copy()
    vc = c["v_cache"].view(torch.int16).numpy().view(np.uint16).copy()
    lens = c["lens_init"].numpy().copy()
    exp_k, exp_v = kc.copy(), vc.copy()
    for t in range(w.steps):
        kn = c["k_new"][t].view(torch.int16).numpy().view(np.uint16).copy()
        vn = c["v_new"][t].view(torch.int16).numpy().view(np.uint16).copy()
        for b in range(w.B):
            exp_k[b, :, lens[b] + 0] = kn[b]
            exp_v[b, :, lens[b] + 0] = vn[b]
        before = lens.copy()
        oracle.kv_append(kc, vc, lens, kn, vn)
        assert np.array_equal(lens, before + 1)
    assert np.array_equal(kc, exp_k) and np.array_equal(vc, exp_v)


@pytest.mark.parametrize("h_q,h_kv,kv", [(1, 1, "f32"), (8, 2, "bf16"), (4, 1, "fp8"), (1, 1, "int8")])
def test_traffic_formula_by_counting_reads(h_q, h_kv, kv):
    """I6 (page "MoA-Structured Decode Attention", §2 memory traffic
    (d_k + n d_k + n d_v + d_v) x bytes; §6 traffic falls by h_q / h_kv): the distinct
    elements the oracle's loops read are exactly q, and the first n rows of K and V of
    each selected group, once."""
    w = workloads.Workload("tr", 2, h_q, h_kv, 8, 30, "bf16" if kv in workloads.SCALED else kv, kv,
                           ("uniform", 1, 30), 0, 3, 0.3)
    c = workloads.generate(w)
    out, (qm, km, vm) = oracle.decode_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"],
                                          w.scale, kv_scales=c["kv_scales"], marks=True)
    d = w.d
    eb = workloads.ELEM_BYTES[kv]
    qb = workloads.ELEM_BYTES[w.q_dtype]
    for b in range(w.B):
        n = int(c["lens_final"][b])
        assert km[b].sum() == h_kv * n * d and vm[b].sum() == h_kv * n * d
        assert km[b, :, :n].all() and vm[b, :, :n].all()
        if h_q == h_kv == 1:  # the single-head formula, element sizes per R15
            bytes_read = int(qm[b].sum()) * qb + int(km[b].sum() + vm[b].sum()) * eb
            assert bytes_read + d * 4 == d * qb + n * d * eb + n * d * eb + d * 4
    assert qm.all()
    assert np.isfinite(out).all()


def test_fp8_e4m3fn_decoder_all_codes():
    """I7: the oracle's own e4m3fn decoder equals torch's cast for all 256 codes."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3fn_to_f64(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got[[0x7F, 0xFF]]).all() and np.isnan(got).sum() == 2
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_int8_decoder_all_codes():
    """The oracle's int8 decoder is the two's-complement value of the byte, for all 256 codes
    (torch's integer cast as the independent check)."""
    codes = torch.arange(-128, 128, dtype=torch.int32).to(torch.int8)
    ref = codes.to(torch.float64).numpy()
    got = np.array([oracle.int8_to_f64(c) for c in range(-128, 128)])
    assert np.array_equal(got, ref)
    assert got[0] == -128.0 and got[-1] == 127.0 and got[128] == 0.0


def test_bf16_decoder_all_codes():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_f64(b) for b in range(0, 65536, 97)])
    r = ref[::97]
    assert np.array_equal(np.isnan(got), np.isnan(r))
    assert np.array_equal(got[~np.isnan(r)], r[~np.isnan(r)])


def test_empty_sequence_is_rejected():
    """R9: softmax over zero rows is undefined; the oracle refuses n = 0."""
    w, c = _rand_case(3)
    lens = c["lens_final"].clone()
    lens[0] = 0
    with pytest.raises(ValueError):
        oracle.decode_f64(c["q"], c["k_cache"], c["v_cache"], lens, w.scale)


def test_thread_count_does_not_change_bits():
    """Parallelism over heads never changes a head's summation order."""
    w, c = _rand_case(23, B=3, h_q=8, h_kv=4, d=64, cap=300, kv="bf16")
    a = oracle.decode_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale, nthreads=1)
    b = oracle.decode_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale, nthreads=4)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- multi-query causal decode
def _mq_case(seed, kv, T, h_q, h_kv, d, cap, lens=None):
    w = workloads.Workload("mq", 3, h_q, h_kv, d, cap, "bf16" if kv in workloads.SCALED else kv, kv,
                           lens or ("uniform", T, cap), 0, seed, 0.7, nq=T)
    c = workloads.generate(w, poison=True)
    if T == 1:
        c["q"] = c["q"][:, None]  # [B, 1, h_q, d]
    return w, c


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8", "int8"])
def test_multi_query_vs_masked_brute_force(seed, kv):
    """Multi-query causal decode against 50-digit masked attention over the whole cache
    (scores + 0 / minus-infinity mask, the forward form of page "Phase 3, Section 6:
    StoryLM-0 head-parallel attention", §3): tiny GQA cases, T = 1..3, ragged lengths >= T."""
    rng = np.random.default_rng(700 + 10 * seed + len(kv))
    T = int(rng.integers(1, 4))
    h_kv = int(rng.integers(1, 3))
    w, c = _mq_case(900 + seed, kv, T, h_kv * int(rng.integers(1, 3)), h_kv, int(rng.integers(1, 5)), 7)
    got = oracle.decode_multi_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale,
                                  kv_scales=c["kv_scales"])
    sc = c["kv_scales"]
    ref = brute.decode_multi(_widen(c["q"]).tolist(), _widen(c["k_cache"], sc, 0).tolist(),
                             _widen(c["v_cache"], sc, 1).tolist(), c["lens_final"].tolist(),
                             float(np.float32(w.scale)))
    np.testing.assert_allclose(got, np.array(ref, dtype=np.float64), rtol=0, atol=1e-13)


@pytest.mark.parametrize("T,h_q,h_kv,d,kv", [
    (4, 32, 8, 128, "bf16"), (2, 8, 1, 64, "f32"), (8, 4, 4, 64, "bf16"), (3, 16, 2, 128, "fp8"),
    (5, 8, 2, 128, "int8")])
def test_multi_query_vs_torch_sdpa_with_causal_mask(T, h_q, h_kv, d, kv):
    """torch SDPA in fp64 on the CPU with an explicit boolean mask: query t of a sequence of
    L rows sees key rows 0 .. L - T + t (its own position and before). GQA by repeat_interleave."""
    w, c = _mq_case(31 + T, kv, T, h_q, h_kv, d, 300)
    got = oracle.decode_multi_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale,
                                  kv_scales=c["kv_scales"])
    sc = c["kv_scales"]
    K = torch.from_numpy(_widen(c["k_cache"], sc, 0))
    V = torch.from_numpy(_widen(c["v_cache"], sc, 1))
    q = c["q"].to(torch.float64)
    for b in range(w.B):
        L = int(c["lens_final"][b])
        kb = K[b, :, :L].repeat_interleave(w.g, dim=0)[None]
        vb = V[b, :, :L].repeat_interleave(w.g, dim=0)[None]
        mask = torch.arange(L)[None, :] <= (L - T + torch.arange(T))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[b].transpose(0, 1)[None], kb, vb, attn_mask=mask, scale=float(np.float32(w.scale)))
        np.testing.assert_allclose(got[b], ref[0].transpose(0, 1).numpy(), rtol=0, atol=1e-12)


def test_multi_query_reduces_to_single_query_decode():
    """T = 1 is the single-query decode, and query t of T is the single-query decode of the
    sequence cut after its own row (lens - T + 1 + t rows): bitwise, in fp64."""
    w, c = _mq_case(5, "bf16", 1, 8, 2, 64, 200)
    one = oracle.decode_multi_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale)
    ref = oracle.decode_f64(c["q"][:, 0], c["k_cache"], c["v_cache"], c["lens_final"], w.scale)
    assert np.array_equal(one[:, 0], ref)
    T = 4
    w, c = _mq_case(6, "bf16", T, 8, 2, 64, 200)
    allq = oracle.decode_multi_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale)
    for t in range(T):
        ref = oracle.decode_f64(c["q"][:, t].contiguous(), c["k_cache"], c["v_cache"],
                                c["lens_final"] - T + 1 + t, w.scale)
        assert np.array_equal(allq[:, t], ref)


def test_multi_query_needs_T_rows():
    w, c = _mq_case(7, "f32", 3, 2, 1, 8, 20)
    lens = c["lens_final"].clone()
    lens[1] = 2
    with pytest.raises(ValueError):
        oracle.decode_multi_f64(c["q"], c["k_cache"], c["v_cache"], lens, w.scale)
