"""Host logic of bench.py, no GPU: the one-GPU guard, the lookup of profiled traffic by the
device-code digest, and the number of rotating cache copies."""
import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _recorded_digest(workload: str) -> str:
    text = open(os.path.join(ROOT, "profiles", f"split_kv_attn__{workload}__pmc.txt")).read()
    return re.search(r"^source_sha256:\s*(\S+)\s*$", text, re.M).group(1)


def test_profiled_traffic_only_for_the_code_it_was_taken_on(monkeypatch):
    digest = _recorded_digest("gqa8_bf16")
    monkeypatch.setattr(bench, "source_sha", lambda: digest)
    traffic = bench.profiled_traffic("gqa8_bf16")
    assert traffic is not None and traffic > 1e9
    monkeypatch.setattr(bench, "source_sha", lambda: "0" * 64)
    assert bench.profiled_traffic("gqa8_bf16") is None
    assert bench.profiled_traffic("no_such_workload") is None


def test_code_digest_ignores_where_the_repository_sits(monkeypatch):
    from decode_attention_kv_split_amd import build
    here = build.code_digest()
    assert re.fullmatch(r"[0-9a-f]{64}", here)
    elsewhere = "/elsewhere/repo"
    monkeypatch.setattr(build, "FLAGS", [f.replace(build.ROOT, elsewhere) for f in build.FLAGS])
    monkeypatch.setattr(build, "ROOT", elsewhere)
    assert build.code_digest() == here
    monkeypatch.setattr(build, "FLAGS", build.FLAGS + ["-O0"])
    assert build.code_digest() != here


def test_cache_rotations():
    gib = 1 << 30
    # at least 2 GiB across the copies, 2 to 8 of them
    assert bench.cache_rotations(2 * gib, 10, 100, False) == 2
    assert bench.cache_rotations(gib // 4, 10, 100, False) == 8
    assert bench.cache_rotations(gib // 100, 10, 100, False) == 8
    # with appends, enough copies that no sequence fills up: room for 865 appends per copy (the
    # timed steps run twice: the two-stage form, then the one-call form)
    for warmup, steps in [(10, 100), (100, 1000), (10, 3000), (100, 12000)]:
        r = bench.cache_rotations(2 * gib, warmup, steps, False, room=865)
        assert bench.uses_per_copy(r, warmup, steps, False) <= 865
        assert r == 2 or bench.uses_per_copy(r - 1, warmup, steps, False) > 865
    # graph replays append once per copy per replay
    assert bench.uses_per_copy(2, 10, 100, True) == 105 + 50
    assert bench.uses_per_copy(2, 10, 100, False, one_call=False) == 55


def test_code_digest_keeps_comments_and_layout_out():
    from decode_attention_kv_split_amd import build
    a = build._code_tokens('int a = 1; // note\n/* block */ const char *s = "x // y /* z */";\n')
    b = build._code_tokens('int a = 1;\n  const char *s = "x // y /* z */";  // other note')
    assert a == b == 'int a = 1; const char *s = "x // y /* z */";'
    assert build._code_tokens("int a = 2;") != build._code_tokens("int a = 1;")
    assert build._code_tokens("char c = '/'; // x") == "char c = '/';"


def test_head_count_override_must_divide_into_groups():
    # checked before any device is touched
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--h-q", "33"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "not a multiple of h_kv" in r.stderr


def test_cpu_baseline_fills_its_budget_with_whole_passes():
    """A batch the oracle finishes well inside the budget is timed over repeated passes of the
    same step, so the baseline rests on about the budget's worth of CPU work."""
    import workloads
    w = workloads.WORKLOADS["gqa8_bf16"].resized(B=2, lens=("const", 64), cap=64, steps=0)
    kv_bytes = 2 * 64 * w.h_kv * 2 * w.d * 2
    r = bench.cpu_baseline(w, 0.3, kv_bytes)
    assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1
    assert r["passes"] > 1 and f"{r['passes']} passes" in r["sample"]
    # whole passes until the budget is reached (the last pass may run past it)
    assert float(r["sample"].rsplit(", ", 1)[1].rstrip(" s")) >= 0.3 * 0.9


def test_lse_parts_take_a_workload_without_an_append():
    # the shard form (decode_attn_run_lse + the merge) has no fused append: refused before any device is touched
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--lse-parts", "8"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "without an append" in r.stderr
