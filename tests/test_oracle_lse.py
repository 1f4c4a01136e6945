"""Pins of the oracle's shard functions: attention over one part of the rows with its
log-sum-exp (oracle.decode_lse_f64) and the log-sum-exp merge of parts (oracle.merge_lse).

Page "MoA-Structured Decode Attention", §2 eq. (2): Step II normalises the exponentials of
the scores by their sum, so attention over a union of disjoint row sets is the combination of
the sets' own results weighted by exp(lse_set), lse = ln sum_l exp(s[l]). The pins below hold
those functions to a 50-digit brute force, to scipy's logsumexp, to closed forms, and to the
whole-sequence decode (itself pinned in test_oracle.py). Everything runs on the CPU.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import brute
import workloads
from tests.test_oracle import _widen


def _case(seed, kv="f32", B=3, h_q=4, h_kv=2, d=8, cap=12, lo=0, T=1):
    w = workloads.Workload("lse", B, h_q, h_kv, d, cap, "f32" if kv == "f32" else "bf16", kv,
                           ("uniform", max(lo, 1), cap), 0, seed, 0.4, nq=T)
    c = workloads.generate(w, poison=False)
    return w, c


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8", "int8"])
def test_lse_vs_decimal_brute_force(seed, kv):
    """Tiny cases, one sequence of them empty, against 50-digit arithmetic (out and lse)."""
    rng = np.random.default_rng(7 * seed + len(kv))
    d = int(rng.integers(1, 5))
    w, c = _case(300 + seed, kv, B=3, h_q=2 * int(rng.integers(1, 3)), h_kv=2, d=d, cap=8)
    lens = c["lens_final"].clone()
    lens[seed % 3] = 0
    out, lse = oracle.decode_lse_f64(c["q"], c["k_cache"], c["v_cache"], lens, w.scale, kv_scales=c["kv_scales"])
    sc = c["kv_scales"]
    K, V = _widen(c["k_cache"], sc, 0), _widen(c["v_cache"], sc, 1)
    ref_o, ref_l = brute.decode_lse(_widen(c["q"]).tolist(), K.tolist(), V.tolist(), lens.tolist(),
                                    float(np.float32(w.scale)))
    np.testing.assert_allclose(out, np.array(ref_o, dtype=np.float64), rtol=0, atol=1e-13)
    ref_l = np.array([[float(x) for x in r] for r in ref_l])
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    np.testing.assert_allclose(lse[fin], ref_l[fin], rtol=0, atol=1e-13)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_lse_vs_scipy_logsumexp(kv):
    """lse against scipy.special.logsumexp of the scores, taken from torch-widened inputs."""
    w, c = _case(41, kv, B=3, h_q=8, h_kv=2, d=64, cap=300)
    out, lse = oracle.decode_lse_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale,
                                     kv_scales=c["kv_scales"])
    sc = c["kv_scales"]
    K, q = _widen(c["k_cache"], sc, 0), _widen(c["q"])
    for b in range(w.B):
        n = int(c["lens_final"][b])
        for h in range(w.h_q):
            s = float(np.float32(w.scale)) * (K[b, h // w.g, :n] @ q[b, h])
            assert abs(lse[b, h] - scipy.special.logsumexp(s)) <= 1e-12 * max(1.0, abs(lse[b, h]))


def test_lse_single_row_is_its_score():
    """One row: the softmax weight is 1, so out is that V row and lse the row's score."""
    w, c = _case(5, "f32", B=2, h_q=4, h_kv=1, d=16, cap=4)
    lens = torch.ones(w.B, dtype=torch.int32)
    out, lse = oracle.decode_lse_f64(c["q"], c["k_cache"], c["v_cache"], lens, w.scale)
    q, K, V = (x.to(torch.float64).numpy() for x in (c["q"], c["k_cache"], c["v_cache"]))
    for b in range(w.B):
        for h in range(w.h_q):
            assert np.array_equal(out[b, h], V[b, 0, 0])
            s = float(np.float32(w.scale)) * math.fsum(q[b, h] * K[b, 0, 0])
            assert abs(lse[b, h] - s) <= 1e-14 * max(1.0, abs(s))


def test_lse_outputs_equal_the_decode_functions():
    """out of the shard function is the decode's own result, bit for bit (T = 1 and T > 1)."""
    w, c = _case(8, "bf16", B=3, h_q=8, h_kv=2, d=32, cap=64)
    out, _ = oracle.decode_lse_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale)
    assert np.array_equal(out, oracle.decode_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale))
    w, c = _case(9, "bf16", B=3, h_q=8, h_kv=2, d=32, cap=64, lo=4, T=4)
    out, _ = oracle.decode_lse_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale)
    ref = oracle.decode_multi_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale)
    assert np.array_equal(out, ref)


def split_rows(c, cuts):
    """The caches cut into parts by row: part p holds rows [cuts[b][p], cuts[b][p+1]) of
    sequence b as a cache of its own (lens = part length, possibly 0)."""
    k, v = c["k_cache"], c["v_cache"]
    B, h_kv, cap, d = k.shape
    parts = []
    for p in range(len(cuts[0]) - 1):
        lens = torch.tensor([cuts[b][p + 1] - cuts[b][p] for b in range(B)], dtype=torch.int32)
        cp = max(1, int(lens.max()))
        kp = torch.zeros((B, h_kv, cp, d), dtype=k.dtype)
        vp = torch.zeros((B, h_kv, cp, d), dtype=v.dtype)
        for b in range(B):
            n = int(lens[b])
            kp[b, :, :n] = k[b, :, cuts[b][p]:cuts[b][p] + n]
            vp[b, :, :n] = v[b, :, cuts[b][p]:cuts[b][p] + n]
        parts.append((kp, vp, lens))
    return parts


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("kv", ["f32", "bf16", "int8"])
def test_merge_of_row_parts_equals_the_whole(seed, kv):
    """Cut every sequence's rows into P parts at random places (empty parts included), attend
    over each part, merge: the result is the attention over all the rows."""
    rng = np.random.default_rng(seed)
    w, c = _case(60 + seed, kv, B=4, h_q=8, h_kv=2, d=16, cap=90)
    P = int(rng.integers(2, 6))
    lens = c["lens_final"].tolist()
    cuts = [[0] + sorted(int(x) for x in rng.integers(0, n + 1, P - 1)) + [n] for n in lens]
    outs, lses = [], []
    for kp, vp, lp in split_rows(c, cuts):
        o, l = oracle.decode_lse_f64(c["q"], kp, vp, lp, w.scale, kv_scales=c["kv_scales"])
        outs.append(o)
        lses.append(l)
    out, lse = oracle.merge_lse(np.stack(outs), np.stack(lses))
    ref_o, ref_l = oracle.decode_lse_f64(c["q"], c["k_cache"], c["v_cache"], c["lens_final"], w.scale,
                                         kv_scales=c["kv_scales"])
    np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-12)


def test_merge_closed_forms():
    """One part: unchanged, bit for bit. An extra empty part (lse -inf): unchanged. The same
    part twice: the same out, lse + ln 2. Parts in another order: the same result. No part
    holding a row: out 0, lse -inf."""
    rng = np.random.default_rng(3)
    o = rng.standard_normal((3, 5, 8))
    l = rng.standard_normal((3, 5)) * 4
    out, lse = oracle.merge_lse(o[None], l[None])
    assert np.array_equal(out, o) and np.array_equal(lse, l)
    out2, lse2 = oracle.merge_lse(np.stack([o, np.zeros_like(o)]), np.stack([l, np.full_like(l, -np.inf)]))
    assert np.array_equal(out2, o) and np.array_equal(lse2, l)
    out3, lse3 = oracle.merge_lse(np.stack([o, o]), np.stack([l, l]))
    np.testing.assert_allclose(out3, o, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse3, l + math.log(2), rtol=0, atol=1e-14)
    o2, l2 = rng.standard_normal((3, 5, 8)), rng.standard_normal((3, 5))
    a = oracle.merge_lse(np.stack([o, o2]), np.stack([l, l2]))
    b = oracle.merge_lse(np.stack([o2, o]), np.stack([l2, l]))
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-15)
    out4, lse4 = oracle.merge_lse(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf))
    assert np.array_equal(out4, np.zeros((3, 4))) and np.all(np.isneginf(lse4))
    # the weights are exp(lse_p - M) / sum: a part far below the others weighs nothing
    out5, lse5 = oracle.merge_lse(np.stack([o, o2]), np.stack([l, l - 800.0]))
    np.testing.assert_allclose(out5, o, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse5, l, rtol=0, atol=1e-15)


def test_empty_and_short_lengths():
    """lens = 0 is an empty part (out 0, lse -inf); 0 < lens < T is refused."""
    w, c = _case(12, "f32", B=2, h_q=2, h_kv=1, d=4, cap=10, lo=3, T=3)
    lens = c["lens_final"].clone()
    lens[0] = 0
    out, lse = oracle.decode_lse_f64(c["q"], c["k_cache"], c["v_cache"], lens, w.scale)
    assert np.array_equal(out[0], np.zeros_like(out[0])) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))
    lens[1] = 2
    with pytest.raises(ValueError):
        oracle.decode_lse_f64(c["q"], c["k_cache"], c["v_cache"], lens, w.scale)
