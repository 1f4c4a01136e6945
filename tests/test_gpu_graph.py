"""The decode loop replayed from a captured HIP graph.

A decode loop captures one fused step (append, attend, combine) once and replays it step after
step: the lengths live on the device, so each replay appends the row the host has just put in
the step's input buffers and attends one row further. Every replay must give the bits that the
same call made eagerly gives on an identical cache (the kernels are deterministic and take the
partition from the device lengths), and the CPU oracle's result within the cache type's
tolerance. Eager torch work (the copies of the next rows and of the output) and a
synchronisation sit between the replays, as in a real loop. No call of the library records a
memset: the workspace is cleared by its own kernels.

The second test replays a captured multi-query attend (no append) with new queries written
between the replays. The third replays one device's shares of a context split in two
(decode_attn_run_lse on each) and their merge.
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
STEPS = 5


def draw(kv, shape, gen):
    """Seeded cache-type values: N(0, 1) rounded for f32 / bf16, every finite code for the
    8-bit types (fp8 without the NaN codes 0x7F / 0xFF, int8 with -128)."""
    if kv == "fp8":
        c = torch.randint(0, 254, shape, generator=gen, dtype=torch.int32)
        return torch.where(c >= 127, c + 1, c).to(torch.uint8).view(torch.float8_e4m3fn)
    if kv == "int8":
        return torch.randint(-128, 128, shape, generator=gen, dtype=torch.int32).to(torch.int8)
    return torch.randn(shape, generator=gen).to(TORCH[kv])


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


CASES = [
    # kv, d, h_q, h_kv, initial lens, cap
    ("bf16", 128, 32, 8, [700, 1, 1200, 64], 1280),      # g = 4, register-ring matrix cores
    ("bf16", 128, 32, 1, [1000, 5, 333], 1100),          # MQA, 32 heads per workgroup
    ("bf16", 64, 4, 4, [300, 900, 1, 64], 1000),         # g = 1, vector ALUs
    ("f32", 64, 1, 1, [1008], 1024),                     # single head, fp32
    ("fp8", 128, 16, 2, [640, 3, 1000, 129], 1100),      # LDS-staged matrix cores
    ("int8", 128, 8, 1, [900, 2, 417], 1000),            # int8, LDS-staged
    ("int8", 64, 6, 2, [640, 1, 999], 1024),             # int8 on the vector ALUs (g = 3)
]


@pytest.mark.parametrize("kv,d,h_q,h_kv,lens,cap", CASES)
def test_graph_replayed_decode_loop(kv, d, h_q, h_kv, lens, cap):
    seed = 500 + CASES.index((kv, d, h_q, h_kv, lens, cap))
    log(f"case graph decode loop {kv} d={d} h_q={h_q} h_kv={h_kv} lens={lens} cap={cap}")
    B = len(lens)
    gen = torch.Generator().manual_seed(seed)
    qd = torch.float32 if kv == "f32" else torch.bfloat16
    q = torch.randn(B, h_q, d, generator=gen).to(qd)
    kc, vc = draw(kv, (B, h_kv, cap, d), gen), draw(kv, (B, h_kv, cap, d), gen)
    kn = [draw(kv, (B, h_kv, d), gen) for _ in range(STEPS)]
    vn = [draw(kv, (B, h_kv, d), gen) for _ in range(STEPS)]
    scales = None
    if kv in ("fp8", "int8"):
        scales = (torch.rand(B, h_kv, 2, generator=gen) * 0.02 + 0.002).to(torch.float32)
    lens0 = torch.tensor(lens, dtype=torch.int32)
    scale = workloads._inv_sqrt(d)
    desc = da.Desc(B, h_q, h_kv, d, cap, qd, TORCH[kv], scale)
    dev = torch.device("cuda")
    qg, sg = q.to(dev), (None if scales is None else scales.to(dev))
    # the graph's state: caches, lengths, the step's input rows, the output
    kgr, vgr, lgr = kc.to(dev), vc.to(dev), lens0.to(dev)
    kin, vin = torch.empty_like(kn[0], device=dev), torch.empty_like(vn[0], device=dev)
    out_g = torch.empty(B, h_q, d, dtype=torch.float32, device=dev)
    ws_g = da.Workspace(desc, cap)
    # the eager path on its own copy
    ke, ve, le = kc.to(dev), vc.to(dev), lens0.to(dev)
    out_e = torch.empty_like(out_g)
    ws_e = da.Workspace(desc, cap)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            da.decode_attn_append_run(desc, qg, kgr, vgr, lgr, kin, vin, cap, sg, out_g, ws_g)
    torch.cuda.synchronize()
    assert torch.equal(lgr.cpu(), lens0), "capturing must not run the step"

    kh, vh = oracle._np(kc).copy(), oracle._np(vc).copy()
    lh = lens0.numpy().copy()
    for t in range(STEPS):
        kin.copy_(kn[t].to(dev))
        vin.copy_(vn[t].to(dev))
        graph.replay()
        got = out_g.clone()
        da.decode_attn_append_run(desc, qg, ke, ve, le, kn[t].to(dev), vn[t].to(dev), cap, sg, out_e, ws_e)
        torch.cuda.synchronize()
        assert np.array_equal(bits(got), bits(out_e)), f"step {t}: graph replay and eager call differ"
        oracle.kv_append(kh, vh, lh, oracle._np(kn[t]).copy(), oracle._np(vn[t]).copy())
        assert lgr.cpu().numpy().tolist() == lh.tolist(), f"step {t}: lengths"
        check_close(got, oracle.decode_f64(q, kh, vh, lh, scale, kv_scales=scales), kv, f"step {t}")
    assert da.da_read_device_error(ws_g) == 0 and da.da_read_device_error(ws_e) == 0
    assert np.array_equal(bits(kgr), kh.view(np.uint8)) and np.array_equal(bits(vgr), vh.view(np.uint8))
    assert np.array_equal(bits(kgr), bits(ke)) and np.array_equal(bits(vgr), bits(ve))


MQ_CASES = [
    # kv, d, h_q, h_kv, T, lens, cap
    ("bf16", 128, 32, 8, 4, [700, 4, 1200, 65], 1280),   # g * T = 16: one 16-row head tile
    ("fp8", 128, 16, 2, 3, [640, 3, 1000], 1024),        # 8-bit codes, g * T = 24
]


@pytest.mark.parametrize("kv,d,h_q,h_kv,T,lens,cap", MQ_CASES)
def test_graph_replayed_multi_query_attend(kv, d, h_q, h_kv, T, lens, cap):
    seed = 600 + MQ_CASES.index((kv, d, h_q, h_kv, T, lens, cap))
    log(f"case graph multi-query {kv} d={d} h_q={h_q} h_kv={h_kv} T={T} lens={lens} cap={cap}")
    B = len(lens)
    gen = torch.Generator().manual_seed(seed)
    qs = [torch.randn(B, T, h_q, d, generator=gen).to(torch.bfloat16) for _ in range(3)]
    kc, vc = draw(kv, (B, h_kv, cap, d), gen), draw(kv, (B, h_kv, cap, d), gen)
    scales = None
    if kv in ("fp8", "int8"):
        scales = (torch.rand(B, h_kv, 2, generator=gen) * 0.02 + 0.002).to(torch.float32)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    scale = workloads._inv_sqrt(d)
    desc = da.Desc(B, h_q, h_kv, d, cap, torch.bfloat16, TORCH[kv], scale, 0, T)
    dev = torch.device("cuda")
    kg, vg, lg = kc.to(dev), vc.to(dev), lens_t.to(dev)
    sg = None if scales is None else scales.to(dev)
    qin = torch.empty(desc.rows_shape(), dtype=torch.bfloat16, device=dev)
    out_g = torch.empty(desc.rows_shape(), dtype=torch.float32, device=dev)
    out_e = torch.empty_like(out_g)
    ws_g, ws_e = da.Workspace(desc, cap), da.Workspace(desc, cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            da.decode_attn_run(desc, qin, kg, vg, lg, cap, sg, out_g, ws_g)
    torch.cuda.synchronize()
    for i, q in enumerate(qs):
        qin.copy_(q.to(dev))
        graph.replay()
        got = out_g.clone()
        da.decode_attn_run(desc, q.to(dev), kg, vg, lg, cap, sg, out_e, ws_e)
        torch.cuda.synchronize()
        assert np.array_equal(bits(got), bits(out_e)), f"replay {i}: graph replay and eager call differ"
        ref = oracle.decode_multi_f64(q, oracle._np(kc), oracle._np(vc), lens_t, scale, kv_scales=scales)
        check_close(got, ref, kv, f"replay {i}")
    assert da.da_read_device_error(ws_g) == 0 and da.da_read_device_error(ws_e) == 0


def test_graph_replayed_context_parts_and_merge():
    """One device's shares of a context split in two, then the merge, captured once and replayed
    with new queries: every replay equals the eager calls bit for bit, and out and lse equal the
    oracle's attention over all the rows."""
    from tests.test_gpu_shard import check_lse
    log("case graph context parts + merge")
    B, h_q, h_kv, d, cap = 3, 32, 1, 128, 900
    gen = torch.Generator().manual_seed(700)
    qs = [torch.randn(B, h_q, d, generator=gen).to(torch.bfloat16) for _ in range(3)]
    kc, vc = draw("bf16", (B, h_kv, 2 * cap, d), gen), draw("bf16", (B, h_kv, 2 * cap, d), gen)
    lens_all = torch.tensor([1700, 901, 40], dtype=torch.int32)
    cut = torch.tensor([900, 450, 0], dtype=torch.int32)  # part 0: rows [0, cut), part 1: the rest
    scale = workloads._inv_sqrt(d)
    desc = da.Desc(B, h_q, h_kv, d, cap, torch.bfloat16, torch.bfloat16, scale)
    dev = torch.device("cuda")
    parts = []
    for p in range(2):
        kp = torch.zeros(B, h_kv, cap, d, dtype=torch.bfloat16)
        vp = torch.zeros_like(kp)
        lp = torch.zeros(B, dtype=torch.int32)
        for b in range(B):
            r0 = 0 if p == 0 else int(cut[b])
            r1 = int(cut[b]) if p == 0 else int(lens_all[b])
            kp[b, :, :r1 - r0] = kc[b, :, r0:r1]
            vp[b, :, :r1 - r0] = vc[b, :, r0:r1]
            lp[b] = r1 - r0
        parts.append((kp.to(dev), vp.to(dev), lp.to(dev)))
    qin = torch.empty(B, h_q, d, dtype=torch.bfloat16, device=dev)
    pouts = torch.empty(2, B, h_q, d, device=dev)
    plses = torch.empty(2, B, h_q, device=dev)
    out_g, lse_g = torch.empty(B, h_q, d, device=dev), torch.empty(B, h_q, device=dev)
    ws = [da.Workspace(desc, cap) for _ in range(2)]
    ws_e = [da.Workspace(desc, cap) for _ in range(2)]

    def step(q, po, pl, out, lse, wss):
        for p, (kp, vp, lp) in enumerate(parts):
            da.decode_attn_run_lse(desc, q, kp, vp, lp, cap, None, po[p], pl[p], wss[p])
        da.decode_attn_merge_lse(po, pl, out, lse)

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(qin, pouts, plses, out_g, lse_g, ws)
    torch.cuda.synchronize()
    po_e, pl_e = torch.empty_like(pouts), torch.empty_like(plses)
    out_e, lse_e = torch.empty_like(out_g), torch.empty_like(lse_g)
    for i, q in enumerate(qs):
        qin.copy_(q.to(dev))
        graph.replay()
        got, got_l = out_g.clone(), lse_g.clone()
        step(q.to(dev), po_e, pl_e, out_e, lse_e, ws_e)
        torch.cuda.synchronize()
        assert np.array_equal(bits(got), bits(out_e)) and np.array_equal(bits(got_l), bits(lse_e)), f"replay {i}"
        ref_o, ref_l = oracle.decode_lse_f64(q, kc, vc, lens_all, scale)
        check_close(got, ref_o, "bf16", f"replay {i}")
        check_lse(got_l, ref_l, f"replay {i} lse")
    for w_ in ws + ws_e:
        assert da.da_read_device_error(w_) == 0
