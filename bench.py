#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X: µs per decode step and achieved HBM GB/s.

A step is one pass of the whole hot path over the workload's batch. For a workload that
appends (the grouped-query one does) it is one decode step, decode_attn_append_run: one
K/V row per (sequence, KV head) is appended and attention runs over the grown cache, the
split-KV attention kernel (which stores the new rows) then the log-sum-exp combine (which
updates the lengths). As in a decode loop the sequences grow by one row per step of their
cache copy, and the bytes of every step are counted at its own lengths. A workload without
an append runs decode_attn_run. Inputs are seeded synthetic tensors (workloads.py) already
resident in HBM when timing starts; R rotating copies of the cache (R * cache bytes >=
2 GiB) keep the 256 MB Infinity Cache from serving one step's reads out of the previous
step's.

Prints ONE JSON line:
  value       = KV-cache bytes per step / wall-clock time per step   (GB/s, 1e9 B/s)
  ms_per_step = wall-clock per step over the timed region, bracketed by synchronisation. The
                timed steps are the step as the product calls it (decode_attn_append_run or
                decode_attn_run, one call), except every event_every-th step, which carries
                the events of `roofline`
  host_issue_us_per_step = host time to issue a step's calls (a step is host-bound when this
                reaches ms_per_step)
  step_us_p10_p50_p90 = a step's time on the GPU's clock (between the starts of consecutive
                event-carrying steps, per step) at the 10th, 50th and 90th percentile
  roofline    = the step's dominant kernel, timed with HIP events on the stream it runs on, in
                every event_every-th timed step: on the split path (two kernels per step) the
                split-KV attention kernel (that step runs in its two-stage form, the partial
                then the combine entry point, with the events around the first); where the
                step is one kernel (the single pass, for small problems) the whole call:
                algorithmic bytes per launch (the KV rows of every sequence plus q) / mean
                launch duration, against the 8 TB/s HBM3E peak; `traffic` is
                the HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE, read
                from the profiles/ summary when it was taken on the current kernel source
  cpu_baseline= the fp64 CPU oracle on the same inputs, full step, host cores
  one_call_form = split path only: the same number of steps again, every one in the one-call
                form (no events inside a step), bracketed by two events
  --lse-parts P = one device's share of a context split P ways (workloads without an append):
                the one-call step is decode_attn_run_lse over this workload's rows (the share,
                e.g. --workload mqa_bf16 --const-len 16384 for 8 parts of 131072 rows), then the
                decode_attn_merge_lse of P part results that follows the all-gather
  stream_ceiling = the read rate of a plain streaming read (da_stream_read over 2 GiB), and
                value and roofline.achieved as percentages of it; measured before the warm-up
                steps, after some 60 ms of untimed streaming that brings the part to steady
                clocks
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "achieved HBM GB/s (KV bytes/step ÷ time, % of peak) + µs/decode step"


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="gqa8_bf16",
                   help="single_head_f32 | mha_bf16 | gqa8_bf16 | mqa_bf16 | gqa8_fp8 | gqa8_int8 | gqa8_mq4_bf16")
    p.add_argument("--const-len", type=int, default=0,
                   help="override: every sequence this long (the 8K/16K/32K sweep)")
    p.add_argument("--h-q", type=int, default=0, help="override: query heads (a group of h_q / h_kv heads)")
    p.add_argument("--h-kv", type=int, default=0, help="override: KV heads")
    p.add_argument("--block-rows", type=int, default=0, help="rows per split (0 = library choice)")
    p.add_argument("--flavour", choices=["auto", "vector", "matrix"], default="auto",
                   help="split-kernel flavour (auto = the library's choice)")
    p.add_argument("--path", choices=["auto", "split", "single"], default="auto",
                   help="launch path of the one-call step (auto = the library's choice)")
    p.add_argument("--rotations", type=int, default=0, help="cache copies to rotate (0 = auto)")
    p.add_argument("--event-every", type=int, default=8,
                   help="events bracket the dominant kernel of every E-th timed step")
    p.add_argument("--graph", action="store_true",
                   help="also time the step replayed from a captured HIP graph (one step per cache copy)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ceiling", action="store_true", help="skip the measured streaming-read ceiling")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle timing budget")
    p.add_argument("--lse-parts", type=int, default=0,
                   help="one device's share of a context split P ways: the one-call step is "
                        "decode_attn_run_lse on this workload (one part's rows, e.g. --const-len L / P), "
                        "then decode_attn_merge_lse of P part results (workloads without an append)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB device copy (FETCH_SIZE / WRITE_SIZE scale factor)")
    return p.parse_args()


def source_sha() -> str:
    """sha256 of the kernel source and its compiler flags (the device code measured)."""
    from decode_attention_kv_split_amd.build import code_digest
    return code_digest()


def profiled_traffic(workload: str):
    """HBM bytes per split-kernel launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source and compiler flags; else None."""
    path = os.path.join(ROOT, "profiles", f"split_kv_attn__{workload}__pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"^\s*([a-z_0-9]+)\s*:\s*(\S+)\s*$", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("source_sha256") != source_sha() or "hbm_bytes_per_launch" not in kv:
        return None
    return float(kv["hbm_bytes_per_launch"])


def split_kernel_name(w, flavour: str = "auto") -> str:
    """The split kernel the library launches for this workload: query groups (g heads times
    the query rows per sequence) of at least 3 rows over a bf16 / fp8 / int8 cache run on the
    matrix cores, unless one flavour is asked for."""
    if flavour == "auto":
        mfma = w.kv_dtype != "f32" and w.h_q // w.h_kv * w.nq >= 3
    else:
        mfma = flavour == "matrix"
    return "split_kv_attn_mfma_kernel" if mfma else "split_kv_attn_kernel"


def stream_ceiling(dev, reps: int = 10, warm_ms: float = 60.0) -> dict:
    """The measured read ceiling: da_stream_read (a plain streaming read, no arithmetic) over a
    2 GiB buffer, 8x the last-level cache, timed with HIP events. Untimed reads first keep the
    part streaming for warm_ms: after idling, its clocks take some 20-30 ms of load to settle
    (a decode step runs 4 % slower in its first 10 ms, an fp8 one 15 %)."""
    import torch
    import decode_attention_kv_split_amd as da
    n = 2 << 30
    buf = torch.zeros(n, dtype=torch.uint8, device=dev)
    sink = torch.empty(512, dtype=torch.float32, device=dev)
    t_end = time.perf_counter() + warm_ms * 1e-3
    while True:
        for _ in range(8):
            da.da_stream_read(buf, sink)
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            break
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream(dev)
    a.record(stream)
    for _ in range(reps):
        da.da_stream_read(buf, sink)
    b.record(stream)
    torch.cuda.synchronize()
    gbs = n * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del buf
    return {"GBs": round(gbs, 1), "bytes": n, "reps": reps, "untimed_warm_ms": warm_ms,
            "kernel": "stream_read_kernel (16-byte non-temporal buffer loads, 512 workgroups)"}


def uses_per_copy(r: int, warmup: int, steps: int, graph: bool, one_call: bool = True) -> int:
    """Steps (warm-up, timed, the one-call loop, graph replays) that use each of r rotating
    cache copies."""
    return -(-(warmup + steps + (steps if one_call else 0)) // r) + (max(1, steps // r) if graph else 0)


def cache_rotations(kv_bytes: int, warmup: int, steps: int, graph: bool, room=None) -> int:
    """Cache copies to rotate: enough that they hold at least 2 GiB (so the 256 MB Infinity
    Cache cannot serve a step from the previous one), 2 to 8; with appends (room = the
    appends a copy takes before its longest sequence is full) more, up to 32, when a long run
    would otherwise fill a sequence."""
    r = max(2, min(8, math.ceil((2 << 30) / max(kv_bytes, 1))))
    if room is not None:
        while uses_per_copy(r, warmup, steps, graph) > room and r < 32:
            r += 1
    return r


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


def main() -> int:
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU sharding is a design note, not built", file=sys.stderr)
        return 2
    import torch

    if args.copy_calibration:
        copy_calibration()
        return 0

    import decode_attention_kv_split_amd as da
    import workloads

    w = workloads.WORKLOADS[args.workload]
    if args.const_len:
        # room past the length for the appends of the run (a cache copy takes one per use)
        room = (args.warmup + 2 * args.steps) + (args.steps if args.graph else 0) + 1 if w.steps else 0
        w = w.resized(lens=("const", args.const_len), cap=max(w.cap, args.const_len + room))
    if args.h_q or args.h_kv:
        w = w.resized(h_q=args.h_q or w.h_q, h_kv=args.h_kv or w.h_kv)
        if w.h_q % w.h_kv:
            print(f"bench.py: h_q {w.h_q} is not a multiple of h_kv {w.h_kv}", file=sys.stderr)
            return 2
    if args.lse_parts and w.steps:
        print("bench.py: --lse-parts takes a workload without an append", file=sys.stderr)
        return 2
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    c = workloads.generate(w, poison=False)
    lens_final = c["lens_final"]
    esz = workloads.ELEM_BYTES[w.kv_dtype]
    row_bytes = w.h_kv * 2 * w.d * esz  # K and V bytes of one row of every KV head
    q_bytes = w.B * w.nq * w.h_q * w.d * workloads.ELEM_BYTES[w.q_dtype]
    cache_bytes = 2 * c["k_cache"].numel() * esz
    appends = w.steps > 0
    # use u of a cache copy (u = step // R) attends over lens_init + 1 + u rows when appending
    lens_first = (c["lens_init"] + 1 if appends else lens_final).to(torch.int64)
    kv_bytes0 = int(lens_first.sum()) * row_bytes
    R = args.rotations or cache_rotations(kv_bytes0, args.warmup, args.steps, args.graph,
                                          w.cap - int(lens_first.max()) + 1 if appends else None)
    graph_reps = max(1, args.steps // R) if args.graph else 0
    uses = uses_per_copy(R, args.warmup, args.steps, args.graph)
    max_len = int(lens_first.max()) + (uses - 1 if appends else 0)
    if max_len > w.cap:
        print(f"bench.py: {uses} appends per cache copy overflow cap {w.cap}; use fewer steps",
              file=sys.stderr)
        return 2

    def step_kv_bytes(i):
        return kv_bytes0 + (w.B * (i // R) * row_bytes if appends else 0)

    flavour = {"auto": da.FLAVOUR_AUTO, "vector": da.FLAVOUR_VECTOR, "matrix": da.FLAVOUR_MATRIX}[args.flavour]
    path = {"auto": da.PATH_AUTO, "split": da.PATH_SPLIT, "single": da.PATH_SINGLE}[args.path]
    desc = da.Desc(w.B, w.h_q, w.h_kv, w.d, w.cap, workloads.TORCH_DTYPE[w.q_dtype],
                   workloads.TORCH_DTYPE[w.kv_dtype], w.scale, args.block_rows, w.nq, flavour, path)
    plan = da.da_plan(desc, max_len)
    # the single pass is one kernel per step; the split path two (split kernel, combine kernel)
    one_kernel = plan["path"] == da.PATH_SINGLE and not args.lse_parts  # the lse form: the split path
    step_kernel = "decode_step_single_kernel" if one_kernel else split_kernel_name(w, args.flavour)
    q = c["q"].to(dev)
    scales = c["kv_scales"].to(dev) if c["kv_scales"] is not None else None
    lens_init = c["lens_init"].to(dev) if appends else lens_final.to(dev)
    k_new = c["k_new"][0].contiguous().to(dev) if appends else None
    v_new = c["v_new"][0].contiguous().to(dev) if appends else None
    slots = []
    k0, v0 = c["k_cache"].to(dev), c["v_cache"].to(dev)
    del c
    for r in range(R):
        kc = k0 if r == 0 else k0.clone()
        vc = v0 if r == 0 else v0.clone()
        slots.append((kc, vc, lens_init.clone() if appends else lens_init))
    ws = da.Workspace(desc, max_len, device=dev)
    out = torch.empty(desc.rows_shape(), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.lse_parts:
        # the share's result with its log-sum-exp, and the P part results the merge takes after an
        # all-gather (zero-filled here: the merge reads and weighs them all the same, whatever the
        # values)
        lse = torch.empty(desc.rows_shape()[:-1], dtype=torch.float32, device=dev)
        parts_out = torch.zeros((args.lse_parts, *desc.rows_shape()), dtype=torch.float32, device=dev)
        parts_lse = torch.zeros((args.lse_parts, *desc.rows_shape()[:-1]), dtype=torch.float32, device=dev)
        merged = torch.empty_like(out)
        merged_lse = torch.empty_like(lse)

    def step(i, ev=None):
        """One step, as the product calls it (one call). With events ev = (a, b) they bracket the
        step's dominant kernel: the whole call on the single pass (one kernel); on the split
        path the step runs in its two-stage form, the split kernel between a and b, then the
        combine."""
        kc, vc, lens = slots[i % R]
        if args.lse_parts and ev is None:
            da.decode_attn_run_lse(desc, q, kc, vc, lens, max_len, scales, out, lse, ws)
            da.decode_attn_merge_lse(parts_out, parts_lse, merged, merged_lse)
            return
        if ev is None or one_kernel:
            if ev is not None:
                ev[0].record(stream)
            if appends:
                da.decode_attn_append_run(desc, q, kc, vc, lens, k_new, v_new, max_len, scales, out, ws)
            else:
                da.decode_attn_run(desc, q, kc, vc, lens, max_len, scales, out, ws)
            if ev is not None:
                ev[1].record(stream)
            return
        ev[0].record(stream)
        if appends:
            da.decode_attn_append_partial(desc, q, kc, vc, lens, k_new, v_new, max_len, scales, ws)
        else:
            da.decode_attn_partial(desc, q, kc, vc, lens, max_len, scales, ws)
        ev[1].record(stream)
        if appends:
            da.decode_attn_append_combine(desc, lens, max_len, out, ws)
        else:
            da.decode_attn_combine(desc, lens, max_len, out, ws)
        if args.lse_parts:
            da.decode_attn_merge_lse(parts_out, parts_lse, merged, merged_lse)

    # the streaming-read ceiling is measured first: its untimed reads also bring the part to
    # steady clocks before the warm-up steps
    ceil = None if args.no_ceiling else stream_ceiling(dev)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    assert da.da_read_device_error(ws) == 0, "device error flagged during warm-up"

    # Every E-th timed step carries the events around its dominant kernel (each event costs the
    # stream a few microseconds: the other steps run as the product calls them, event-free)
    E = max(1, min(args.event_every, args.steps))
    sampled = list(range(E - 1, args.steps, E))  # not the first timed step, which follows a sync
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in sampled]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, evs[i // E] if i % E == E - 1 else None)
    end.record(stream)
    t_issued = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert da.da_read_device_error(ws) == 0, "device error flagged during the timed steps"

    one_call = None
    if not one_kernel:
        # the same number of steps, every one in the one-call form (no events inside a step),
        # to show what the event-carrying steps cost
        o0, o1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        base = args.warmup + args.steps
        torch.cuda.synchronize()
        o0.record(stream)
        for i in range(args.steps):
            step(base + i)
        o1.record(stream)
        torch.cuda.synchronize()
        assert da.da_read_device_error(ws) == 0, "device error flagged during the one-call steps"
        o_ms = o0.elapsed_time(o1) / args.steps
        o_bytes = sum(step_kv_bytes(base + i) for i in range(args.steps)) / args.steps
        one_call = {"us_per_step": round(o_ms * 1e3, 2), "GBs": round(o_bytes / (o_ms * 1e-3) / 1e9, 2),
                    "steps": args.steps}

    graph = None
    if args.graph:
        # one step per cache copy captured on a side stream, replayed graph_reps times; the
        # lengths live on the device, so every replay appends and attends one row further
        base = args.warmup + 2 * args.steps
        base += (-base) % R  # the next step of copy 0
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for r in range(R):
                    step(base + r)
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(graph_reps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        assert da.da_read_device_error(ws) == 0, "device error flagged during the graph replays"
        n = graph_reps * R
        g_ms = g0.elapsed_time(g1) / n
        g_bytes = sum(step_kv_bytes(base + i) for i in range(n)) / n
        graph = {"us_per_step": round(g_ms * 1e3, 2), "GBs": round(g_bytes / (g_ms * 1e-3) / 1e9, 2),
                 "steps": n, "launch": "HIP graph of one step per cache copy, replayed"}

    timed = range(args.warmup, args.warmup + args.steps)
    kv_bytes = sum(step_kv_bytes(i) for i in timed) / args.steps  # mean over the timed steps
    wall_ms = (t1 - t0) * 1e3 / args.steps
    gpu_ms = start.elapsed_time(end) / args.steps
    # a step's time on the GPU's clock: between consecutive sampled starts, per step
    starts = [a for a, _ in evs] + [end]
    step_sorted = sorted(starts[j].elapsed_time(starts[j + 1]) / (min(args.steps, sampled[j] + E) - sampled[j])
                         for j in range(len(sampled)))
    split_ms = [a.elapsed_time(b) for a, b in evs]
    split_ms_mean = sum(split_ms) / len(split_ms)
    split_sorted = sorted(split_ms)
    algo_bytes = kv_bytes + q_bytes
    achieved = algo_bytes / (split_ms_mean * 1e-3) / 1e9
    value = kv_bytes / (wall_ms * 1e-3) / 1e9
    traffic = (profiled_traffic(args.workload)
               if not (args.const_len or args.block_rows or args.h_q or args.h_kv) and args.flavour == "auto"
               and args.path == "auto" else None)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "us_per_step": round(wall_ms * 1e3, 2),
        "gpu_event_us_per_step": round(gpu_ms * 1e3, 2),
        "host_issue_us_per_step": round((t_issued - t0) * 1e6 / args.steps, 2),
        "step_us_p10_p50_p90": [round(step_sorted[(k * len(step_sorted)) // 10] * 1e3, 2) for k in (1, 5, 9)],
        "event_every": E,
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.B, "h_q": w.h_q, "h_kv": w.h_kv, "head_dim": w.d,
            "cap": w.cap, "q_dtype": w.q_dtype, "kv_dtype": w.kv_dtype, "query_rows_per_seq": w.nq,
            "lens": (f"const {int(lens_final.max())}" if w.lens[0] == "const"
                     else f"uniform[{w.lens[1]},{w.lens[2]}] seed {w.seed}"),
            "sum_lens_first_step": int(lens_first.sum()), "max_len": max_len,
            "appends_per_step": int(appends), "kv_bytes_per_step": round(kv_bytes),
            "rotations": R, "cache_bytes_per_copy": cache_bytes, "flavour": args.flavour,
            **{k: v for k, v in plan.items() if k != "path"},
            "path": "single" if one_kernel else "split",
            **({"lse_parts": args.lse_parts,
                "step": "decode_attn_run_lse on this share, then decode_attn_merge_lse of the parts"}
               if args.lse_parts else {}),
        },
        "roofline": {
            "kernel": step_kernel,
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": round(algo_bytes),
            "launch_us_mean": round(split_ms_mean * 1e3, 2),
            "launch_us_p10": round(split_sorted[len(split_sorted) // 10] * 1e3, 2),
            "launch_us_p90": round(split_sorted[(9 * len(split_sorted)) // 10] * 1e3, 2),
        },
        "cpu_baseline": None,
    }
    if graph is not None:
        result["graph_replay"] = graph
    if one_call is not None:
        result["one_call_form"] = one_call
    if ceil is not None:
        ceil["value_pct_of_ceiling"] = round(100 * value / ceil["GBs"], 2)
        ceil["achieved_pct_of_ceiling"] = round(100 * achieved / ceil["GBs"], 2)
        result["stream_ceiling"] = ceil
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, kv_bytes0)
    print(json.dumps(result), flush=True)
    return 0


def cpu_baseline(w, budget_s: float, kv_bytes_full: int) -> dict:
    """The fp64 oracle, unchanged, on the host cores: whole sequences of the same workload
    (the first k sequences, k chosen to fit the time budget), caches after the append."""
    import numpy as np
    import torch

    import oracle
    import workloads

    nthreads = int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)
    c = workloads.generate(w, poison=False)
    kc = oracle._np(c["k_cache"]).copy() if w.steps else oracle._np(c["k_cache"])
    vc = oracle._np(c["v_cache"]).copy() if w.steps else oracle._np(c["v_cache"])
    lens = c["lens_init"].numpy().copy()
    for t in range(w.steps):
        oracle.kv_append(kc, vc, lens, oracle._np(c["k_new"][t]).copy(), oracle._np(c["v_new"][t]).copy())
    esz = workloads.ELEM_BYTES[w.kv_dtype]
    # time one sequence first, then grow the sample to about the budget
    order = list(range(w.B))
    per_seq = []

    def run(bs):
        sl = slice(bs[0], bs[-1] + 1)
        sc = None if c["kv_scales"] is None else c["kv_scales"][sl].contiguous()
        t = time.perf_counter()
        fn = oracle.decode_multi_f64 if w.nq > 1 else oracle.decode_f64
        fn(c["q"][sl].contiguous(), np.ascontiguousarray(kc[sl]), np.ascontiguousarray(vc[sl]),
           lens[sl], w.scale, kv_scales=sc, nthreads=nthreads)
        return time.perf_counter() - t

    t_one = run([0])
    est_per_row = t_one / max(int(lens[0]), 1)
    k = 1
    while k < w.B and est_per_row * float(lens[:k + 1].sum()) <= budget_s:
        k += 1
    elapsed = run(order[:k])
    passes = 1
    if k == w.B:  # the whole batch is under the budget: the same step again, until it is reached
        while elapsed < budget_s and passes < 10000:
            elapsed += run(order[:k])
            passes += 1
    rows = int(lens[:k].sum())
    sample_bytes = rows * w.h_kv * 2 * w.d * esz * passes
    gbs = sample_bytes / elapsed / 1e9
    full_step_s = elapsed * (kv_bytes_full / sample_bytes)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "sample": f"first {k} of {w.B} sequences ({rows} rows x {w.h_kv} KV heads, all "
                      f"{w.h_q} query heads" + (f" x {w.nq} query rows" if w.nq > 1 else "") +
                      f"), fp64, {passes} pass{'es' if passes > 1 else ''}, {elapsed:.2f} s",
            "passes": passes,
            "us_per_full_step_est": round(full_step_s * 1e6, 1),
            "cpu": _cpu_model()}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    sys.exit(main())
