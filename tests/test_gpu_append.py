"""The fused decode step (decode_attn_append_run and its two stages) on the GPU.

It must give exactly what kv_append followed by decode_attn_run gives: the same output
bits, the same cache bytes, the same lengths and the same error word (the two paths run the
same arithmetic on the same bytes; only where the appended row is read from differs). The
cases cover every kernel flavour and cache type, a new row read by two workgroups (two head
tiles per KV head), 64-byte 8-bit rows (a cache line shared by two rows), a full sequence whose append is
skipped, an empty sequence that the append makes one row long, and small workgroup shares
(many segments). The output is also checked against the CPU oracle.
"""
import numpy as np
import pytest
import torch

import decode_attention_kv_split_amd as da
import oracle
import workloads
from tests.gpu_case import check_close, log

pytestmark = pytest.mark.gpu

TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn, "int8": torch.int8}


def make_case(kv, d, h_q, h_kv, lens, cap, seed):
    """Seeded caches filled at every row (no poison: a full sequence attends over all of cap),
    new rows, q, and slot scales for 8-bit caches."""
    gen = torch.Generator().manual_seed(seed)
    B = len(lens)
    qd = torch.float32 if kv == "f32" else torch.bfloat16
    q = torch.randn(B, h_q, d, generator=gen).to(qd)
    if kv == "fp8":
        def codes(shape):  # every finite e4m3fn code but 0x7F / 0xFF (NaN)
            c = torch.randint(0, 254, shape, generator=gen, dtype=torch.int32)
            c = torch.where(c >= 127, c + 1, c)
            return c.to(torch.uint8).view(torch.float8_e4m3fn)
        kc, vc = codes((B, h_kv, cap, d)), codes((B, h_kv, cap, d))
        kn, vn = codes((B, h_kv, d)), codes((B, h_kv, d))
        scales = (torch.rand(B, h_kv, 2, generator=gen) * 0.02 + 0.002).to(torch.float32)
    elif kv == "int8":
        def codes(shape):  # every code, -128 included
            return torch.randint(-128, 128, shape, generator=gen, dtype=torch.int32).to(torch.int8)
        kc, vc = codes((B, h_kv, cap, d)), codes((B, h_kv, cap, d))
        kn, vn = codes((B, h_kv, d)), codes((B, h_kv, d))
        scales = (torch.rand(B, h_kv, 2, generator=gen) * 0.02 + 0.002).to(torch.float32)
    else:
        kc = torch.randn(B, h_kv, cap, d, generator=gen).to(TORCH[kv])
        vc = torch.randn(B, h_kv, cap, d, generator=gen).to(TORCH[kv])
        kn = torch.randn(B, h_kv, d, generator=gen).to(TORCH[kv])
        vn = torch.randn(B, h_kv, d, generator=gen).to(TORCH[kv])
        scales = None
    return dict(q=q, kc=kc, vc=vc, kn=kn, vn=vn, scales=scales, lens=torch.tensor(lens, dtype=torch.int32))


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def run_both(kv, d, h_q, h_kv, lens, cap, seed, block_rows, path=da.PATH_AUTO):
    c = make_case(kv, d, h_q, h_kv, lens, cap, seed)
    desc = da.Desc(len(lens), h_q, h_kv, d, cap, c["q"].dtype, TORCH[kv], workloads._inv_sqrt(d), block_rows,
                   1, da.FLAVOUR_AUTO, path)
    max_len = cap
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in c.items()}
    sc = g["scales"]
    # path A: kv_append, then decode_attn_run
    ka, va, la = g["kc"].clone(), g["vc"].clone(), g["lens"].clone()
    wsa = da.Workspace(desc, max_len)
    out_a = torch.empty(len(lens), h_q, d, device="cuda")
    da.kv_append(desc, ka, va, la, g["kn"], g["vn"], wsa)
    da.decode_attn_run(desc, g["q"], ka, va, la, max_len, sc, out_a, wsa)
    # path B: the fused step
    kb, vb, lb = g["kc"].clone(), g["vc"].clone(), g["lens"].clone()
    wsb = da.Workspace(desc, max_len)
    out_b = torch.empty_like(out_a)
    da.decode_attn_append_run(desc, g["q"], kb, vb, lb, g["kn"], g["vn"], max_len, sc, out_b, wsb)
    return c, dict(out=out_a, k=ka, v=va, lens=la, err=da.da_read_device_error(wsa)), \
        dict(out=out_b, k=kb, v=vb, lens=lb, err=da.da_read_device_error(wsb))


CASES = [
    # kv, d, h_q, h_kv, lens (cap 1500: 1500 = full, append skipped; 0 becomes one row)
    ("bf16", 128, 8, 2, [1500, 0, 5, 700, 1499, 1]),      # g = 4, matrix cores, 4 heads
    ("bf16", 128, 32, 1, [600, 1499, 3]),                 # MQA, 32 heads per workgroup
    ("bf16", 128, 64, 1, [900, 77, 1499]),                # two head tiles: two readers of a new row
    ("bf16", 64, 4, 4, [300, 1500, 0, 64]),               # g = 1, vector ALUs
    ("f32", 64, 3, 1, [1000, 17, 1499]),                  # fp32, g = 3
    ("fp8", 128, 8, 1, [1200, 33, 0, 1499]),              # fp8, LDS-staged segment
    ("fp8", 64, 16, 2, [640, 1, 1500, 1023]),             # 64-byte rows: two rows per cache line
    ("int8", 128, 8, 1, [1200, 33, 0, 1499]),             # int8, LDS-staged segment
    ("int8", 64, 6, 2, [640, 1, 1500, 1023]),             # int8 on the vector ALUs (g = 3)
]


@pytest.mark.parametrize("block_rows,path", [(0, da.PATH_SPLIT), (37, da.PATH_SPLIT), (0, da.PATH_SINGLE)])
@pytest.mark.parametrize("kv,d,h_q,h_kv,lens", CASES)
def test_fused_step_equals_append_then_run(kv, d, h_q, h_kv, lens, block_rows, path):
    """Both paths of the one-call entry points: the split kernel + combine (library shares or
    37-row shares) and the single pass (one workgroup per sequence, one launch)."""
    seed = 300 + CASES.index((kv, d, h_q, h_kv, lens))
    log(f"case fused append {kv} d={d} h_q={h_q} h_kv={h_kv} lens={lens} block_rows={block_rows} path={path}")
    c, a, b = run_both(kv, d, h_q, h_kv, lens, 1500, seed, block_rows, path)
    assert np.array_equal(bits(a["out"]), bits(b["out"])), "outputs differ"
    assert np.array_equal(bits(a["k"]), bits(b["k"])) and np.array_equal(bits(a["v"]), bits(b["v"]))
    assert torch.equal(a["lens"], b["lens"])
    expect = [L + 1 if L < 1500 else L for L in lens]
    assert b["lens"].cpu().tolist() == expect
    full = any(L >= 1500 for L in lens)
    assert a["err"] == b["err"] == (da.DEV_ERR_APPEND_FULL if full else 0)
    # and both agree with the oracle over the appended caches
    ref = oracle.decode_f64(c["q"], oracle._np(a["k"].cpu()), oracle._np(a["v"].cpu()),
                            np.array(expect, dtype=np.int32), workloads._inv_sqrt(d), kv_scales=c["scales"])
    check_close(b["out"], ref, kv, "fused step")


def test_fused_two_stage_equals_fused_run():
    """decode_attn_append_partial + decode_attn_append_combine = decode_attn_append_run, and
    lens changes only in the combine."""
    kv, d, h_q, h_kv, lens, cap = "bf16", 128, 32, 8, [1000, 1, 2047, 513, 4, 1800], 2048
    c = make_case(kv, d, h_q, h_kv, lens, cap, 377)
    desc = da.Desc(len(lens), h_q, h_kv, d, cap, torch.bfloat16, torch.bfloat16, workloads._inv_sqrt(d), 256)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in c.items()}
    k1, v1, l1 = g["kc"].clone(), g["vc"].clone(), g["lens"].clone()
    ws1 = da.Workspace(desc, cap)
    one = torch.empty(len(lens), h_q, d, device="cuda")
    da.decode_attn_append_run(desc, g["q"], k1, v1, l1, g["kn"], g["vn"], cap, None, one, ws1)
    k2, v2, l2 = g["kc"].clone(), g["vc"].clone(), g["lens"].clone()
    ws2 = da.Workspace(desc, cap)
    two = torch.empty_like(one)
    da.decode_attn_append_partial(desc, g["q"], k2, v2, l2, g["kn"], g["vn"], cap, None, ws2)
    torch.cuda.synchronize()
    assert torch.equal(l2, g["lens"]), "the first stage must not change lens"
    da.decode_attn_append_combine(desc, l2, cap, two, ws2)
    assert da.da_read_device_error(ws1) == 0 and da.da_read_device_error(ws2) == 0
    assert torch.equal(l1, l2) and l2.cpu().tolist() == [L + 1 for L in lens]
    assert np.array_equal(bits(k1), bits(k2)) and np.array_equal(bits(v1), bits(v2))
    assert (one - two).abs().max().item() <= 1e-5


@pytest.mark.parametrize("path", [da.PATH_AUTO, da.PATH_SPLIT])
def test_fused_steps_in_a_loop_match_the_oracle(path):
    """The single-head fp32 workload driven by the fused step alone: 16 steps, n 1008 -> 1024,
    every step within 1e-5 of the oracle and the cache bit-exact at the end; the library's
    choice (the single pass: one launch per step) and the split path."""
    w = workloads.WORKLOADS["single_head_f32"]
    c = workloads.generate(w)
    desc = da.Desc(w.B, w.h_q, w.h_kv, w.d, w.cap, torch.float32, torch.float32, w.scale, 0, 1, da.FLAVOUR_AUTO, path)
    assert da.da_plan(desc, w.cap)["path"] == (da.PATH_SINGLE if path == da.PATH_AUTO else da.PATH_SPLIT)
    kc, vc = c["k_cache"].cuda(), c["v_cache"].cuda()
    lens = c["lens_init"].cuda()
    q = c["q"].cuda()
    ws = da.Workspace(desc, w.cap)
    out = torch.empty(1, 1, w.d, device="cuda")
    kh = oracle._np(c["k_cache"]).copy()
    vh = oracle._np(c["v_cache"]).copy()
    ln = c["lens_init"].numpy().copy()
    for t in range(w.steps):
        da.decode_attn_append_run(desc, q, kc, vc, lens, c["k_new"][t].contiguous().cuda(),
                                  c["v_new"][t].contiguous().cuda(), w.cap, None, out, ws)
        oracle.kv_append(kh, vh, ln, c["k_new"][t].numpy().copy(), c["v_new"][t].numpy().copy())
        check_close(out, oracle.decode_f64(c["q"], kh, vh, ln, w.scale), "f32", f"step {t}")
    assert int(lens.item()) == 1024 and da.da_read_device_error(ws) == 0
    assert np.array_equal(oracle._np(kc.cpu()), kh) and np.array_equal(oracle._np(vc.cpu()), vh)


@pytest.mark.parametrize("kv,d", [("bf16", 128), ("fp8", 128)])
def test_fused_step_on_caches_off_cache_line_alignment(kv, d):
    """Caches whose base is 16-byte but not cache-line aligned (rows then share lines with
    their neighbours): the fused step must still read the new rows it stores."""
    lens, h_q, h_kv, cap = [700, 3, 1499, 64], 8, 2, 1500
    c = make_case(kv, d, h_q, h_kv, lens, cap, 401)
    desc = da.Desc(len(lens), h_q, h_kv, d, cap, c["q"].dtype, TORCH[kv], workloads._inv_sqrt(d), 37)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in c.items()}

    def shifted(t):  # the same values at a base 64 bytes past a cache line
        n = t.numel() * t.element_size()
        raw = torch.zeros(n + 256, dtype=torch.uint8, device="cuda")
        off = (-raw.data_ptr()) % 128 + 64
        view = raw[off:off + n].view(t.dtype).view(t.shape)
        view.copy_(t)
        assert view.data_ptr() % 128 == 64 and view.is_contiguous()
        return view

    kc, vc, ln = shifted(g["kc"]), shifted(g["vc"]), g["lens"].clone()
    ws = da.Workspace(desc, cap)
    out = torch.empty(len(lens), h_q, d, device="cuda")
    da.decode_attn_append_run(desc, g["q"], kc, vc, ln, g["kn"], g["vn"], cap, g["scales"], out, ws)
    assert da.da_read_device_error(ws) == 0
    expect = [L + 1 for L in lens]
    assert ln.cpu().tolist() == expect
    kh, vh = oracle._np(c["kc"]).copy(), oracle._np(c["vc"]).copy()
    l0 = np.array(lens, dtype=np.int32)
    oracle.kv_append(kh, vh, l0, oracle._np(c["kn"]).copy(), oracle._np(c["vn"]).copy())
    assert np.array_equal(oracle._np(kc.cpu()), kh) and np.array_equal(oracle._np(vc.cpu()), vh)
    ref = oracle.decode_f64(c["q"], kh, vh, l0, workloads._inv_sqrt(d), kv_scales=c["scales"])
    check_close(out, ref, kv, "fused step, off-line caches")
