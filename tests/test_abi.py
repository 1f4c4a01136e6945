"""C-ABI checks that need no GPU: the library loads, exports every entry point the
header declares, and rejects invalid arguments on the host before launching anything.

Every call here fails validation (or only does host arithmetic), so no kernel is
launched and no device is touched; fake device addresses are never dereferenced.
"""
import ctypes
import os
import re

import pytest
import torch

import decode_attention_kv_split_amd as da
from decode_attention_kv_split_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decode_attn.h")

FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced on the host


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.library_path()):
        from decode_attention_kv_split_amd import build
        build.build_library()
    return _lib.load()


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} is declared in the header but not exported"


def _desc(**kw):
    base = dict(batch=2, h_q=8, h_kv=2, d_k=128, d_v=128, cap=1024, q_dtype=1, kv_dtype=1,
                scale=0.088, block_rows=0, n_queries=0, flavour=0, path=1)  # the split path's plan
    base.update(kw)
    return da._CDesc(**base)


def _ws_size(lib, desc, max_len):
    n = ctypes.c_size_t(0)
    rc = lib.da_workspace_size(ctypes.byref(desc), max_len, ctypes.byref(n))
    return rc, n.value


@pytest.mark.parametrize("kw,max_len,code", [
    (dict(h_q=6, h_kv=4), 100, -1),           # h_q not a multiple of h_kv
    (dict(batch=0), 100, -1),
    (dict(), 0, -1),                           # max_len < 1
    (dict(), 2000, -1),                        # max_len > cap
    (dict(d_k=96, d_v=96), 100, -2),           # head size not built
    (dict(d_k=128, d_v=64), 100, -2),          # d_k != d_v
    (dict(q_dtype=0, kv_dtype=1), 100, -2),    # dtype pair not built
    (dict(kv_dtype=7), 100, -1),               # unknown dtype code
    (dict(block_rows=-1), 100, -1),            # negative workgroup share
    (dict(batch=1025), 100, -2),               # more sequences than one call takes
    (dict(scale=float("nan")), 100, -1),
    (dict(n_queries=-1), 100, -1),             # negative query rows
    (dict(n_queries=1025), 100, -1),           # more query rows per sequence than one call takes
])
def test_invalid_descriptors_are_rejected(lib, kw, max_len, code):
    rc, _ = _ws_size(lib, _desc(**kw), max_len)
    assert rc == code
    assert lib.da_last_error()  # a message was recorded


def _plan(lib, d, max_len):
    r, n, g = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    assert lib.da_plan(ctypes.byref(d), max_len, ctypes.byref(r), ctypes.byref(n), ctypes.byref(g), None) == 0
    return r.value, n.value, g.value


def test_workspace_size_and_plan(lib):
    """The partition covers every row at max_len; the workspace holds one (max, sum, row)
    slot per segment (workgroups + units) and per head of a workgroup."""
    d = _desc(batch=16, h_q=32, h_kv=8, cap=32768)
    rc, n = _ws_size(lib, d, 32768)
    assert rc == 0
    rows_per_block, nblocks, gt = _plan(lib, d, 32768)
    units = 16 * 8 * (32 // 8 // gt)
    assert gt == 4 and rows_per_block * nblocks >= units * 32768 and rows_per_block >= 256
    segs = nblocks + units
    assert n >= 256 + segs * gt * 2 * 4 + segs * gt * 128 * 4
    d2 = _desc(batch=16, h_q=32, h_kv=8, cap=32768, block_rows=512)
    assert _plan(lib, d2, 1000) == (512, -(-128 * 1000 // 512), 4)
    # query rows per head tile: a group's g query rows in as few tiles as the flavour allows
    # (32 rows on the matrix cores, 8 for fp32 on the vector ALUs), of nearly equal size
    assert _plan(lib, _desc(h_q=6, h_kv=2), 100)[2] == 3
    assert _plan(lib, _desc(h_q=12, h_kv=2), 100)[2] == 6
    assert _plan(lib, _desc(h_q=8, h_kv=2), 100)[2] == 4
    assert _plan(lib, _desc(h_q=64, h_kv=1), 100)[2] == 32
    assert _plan(lib, _desc(h_q=80, h_kv=2), 100)[2] == 20   # 40 rows: two tiles of 20
    assert _plan(lib, _desc(h_q=74, h_kv=2), 100)[2] == 19   # 37 rows: tiles of 19 and 18
    assert _plan(lib, _desc(h_q=64, h_kv=2, q_dtype=0, kv_dtype=0), 100)[2] == 8
    assert _plan(lib, _desc(h_q=18, h_kv=2, q_dtype=0, kv_dtype=0), 100)[2] == 5  # 9 rows: 5 + 4


@pytest.mark.parametrize("g,nq", [(3, 1), (5, 1), (6, 1), (7, 1), (12, 1), (24, 1), (28, 1), (32, 1),
                                  (5, 3), (5, 4), (6, 4), (7, 4), (3, 8), (4, 5), (1, 7)])
def test_one_head_tile_per_group_up_to_32_query_rows(lib, g, nq):
    """Every KV group with g * T <= 32 query rows over a bf16, fp8 or int8 cache is one head
    tile (its K and V rows are read once), whatever g * T's divisors."""
    for kv in (1, 2, 3):
        d = _desc(batch=3, h_q=2 * g, h_kv=2, kv_dtype=kv, n_queries=nq)
        rows_per_block, nblocks, gt = _plan(lib, d, 1000)
        assert gt == g * nq, (kv, g, nq, gt)
        # the partition spans the rows of one tile per (sequence, KV head)
        assert rows_per_block * nblocks >= 3 * 2 * 1000 and (rows_per_block - 1) * nblocks < 3 * 2 * 1000 + nblocks


def test_flavour_override(lib):
    """DA_FLAVOUR_VECTOR / _MATRIX pick one flavour; the matrix cores refuse an fp32 cache."""
    assert _plan(lib, _desc(h_q=32, h_kv=8, flavour=1), 100)[2] == 4   # vector ALUs: tiles of <= 4
    assert _plan(lib, _desc(h_q=48, h_kv=2, flavour=1), 100)[2] == 4   # 24 rows: six tiles of 4
    assert _plan(lib, _desc(h_q=8, h_kv=8, flavour=2), 100)[2] == 1    # one row padded to 16 slots
    assert _ws_size(lib, _desc(q_dtype=0, kv_dtype=0, flavour=2), 100)[0] == -2
    assert _ws_size(lib, _desc(flavour=3), 100)[0] == -1


def test_null_and_misaligned_pointers_fail_before_launch(lib):
    d = _desc()
    assert lib.kv_append(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    assert lib.kv_append(ctypes.byref(d), ctypes.c_void_p(0x10002), FAKE, FAKE, FAKE, FAKE, None, None) == -1
    assert lib.decode_attn_run(ctypes.byref(d), None, FAKE, FAKE, FAKE, 100, None, FAKE, FAKE, 1 << 30, None) == -1
    assert lib.decode_attn_run(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 100, None, None, FAKE, 1 << 30, None) == -1
    fp8 = _desc(kv_dtype=2)
    assert lib.decode_attn_partial(ctypes.byref(fp8), FAKE, FAKE, FAKE, FAKE, 100, None, FAKE, 1 << 30, None) == -1
    assert lib.da_read_device_error(None, None, None) == -1
    assert lib.da_workspace_init(None, 1024, None) == -1
    assert lib.da_workspace_init(FAKE, 16, None) == -3


def test_fused_append_needs_both_new_rows(lib):
    d = _desc()
    args = (ctypes.byref(d), FAKE, FAKE, FAKE, FAKE)
    assert lib.decode_attn_append_run(*args, None, FAKE, 100, None, FAKE, FAKE, 1 << 30, None) == -1
    assert lib.decode_attn_append_run(*args, FAKE, None, 100, None, FAKE, FAKE, 1 << 30, None) == -1
    assert lib.decode_attn_append_run(*args, ctypes.c_void_p(0x10008), FAKE, 100, None, FAKE, FAKE,
                                      1 << 30, None) == -1  # misaligned
    assert lib.decode_attn_append_run(*args, FAKE, FAKE, 100, None, None, FAKE, 1 << 30, None) == -1  # no out
    assert lib.decode_attn_append_partial(*args, FAKE, None, 100, None, FAKE, 1 << 30, None) == -1
    rc, n = _ws_size(lib, d, 1000)
    assert lib.decode_attn_append_combine(ctypes.byref(d), FAKE, 1000, FAKE, FAKE, n - 1, None) == -3


def test_small_workspace_is_rejected(lib):
    d = _desc()
    rc, n = _ws_size(lib, d, 1000)
    assert rc == 0
    assert lib.decode_attn_run(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 1000, None, FAKE, FAKE, n - 1, None) == -3
    assert lib.decode_attn_combine(ctypes.byref(d), FAKE, 1000, FAKE, FAKE, n - 1, None) == -3


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        assert lib.da_status_string(code)
    assert lib.da_status_string(0) == b"ok"
    assert lib.da_status_string(-3) == b"workspace too small"


def test_python_binding_marshalling_errors():
    """The binding refuses CPU tensors and wrong shapes before calling the library."""
    desc = da.Desc(1, 4, 2, 64, 128, torch.bfloat16, torch.bfloat16, 0.125)
    q = torch.zeros(1, 4, 64, dtype=torch.bfloat16)
    kc = torch.zeros(1, 2, 128, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        da.decode_attn_run(desc, q, kc, kc, torch.ones(1, dtype=torch.int32), 1, None,
                           torch.zeros(1, 4, 64), torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(da.DecodeAttnError):
        da.da_workspace_size(da.Desc(1, 3, 2, 64, 128, torch.bfloat16, torch.bfloat16, 0.125), 10)
    with pytest.raises(TypeError):  # the caller chooses the scale: the binding has no default
        da.Desc(1, 4, 2, 64, 128, torch.bfloat16, torch.bfloat16)


def test_int8_cache_is_built_and_needs_scales(lib):
    """(bf16 q, int8 cache) is a supported pair on both flavours; like fp8 it needs kv_scales."""
    for h_q in (8, 6):  # g = 4: matrix cores; g = 3: vector ALUs
        d = _desc(h_q=h_q, kv_dtype=3)
        rc, n = _ws_size(lib, d, 1000)
        assert rc == 0 and n > 0
        assert lib.decode_attn_run(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 1000, None, FAKE, FAKE, n, None) == -1
        assert b"kv_scales" in lib.da_last_error()
    assert _ws_size(lib, _desc(q_dtype=0, kv_dtype=3), 100)[0] == -2  # fp32 q over int8: not built


def test_stream_read_rejects_bad_sizes(lib):
    assert lib.da_stream_read(FAKE, 1000, FAKE, None) == -1          # not a multiple of 16
    assert lib.da_stream_read(ctypes.c_void_p(0x10008), 1024, FAKE, None) == -1  # misaligned
    assert lib.da_stream_read(FAKE, 0, FAKE, None) == -1
    assert lib.da_stream_read(None, 1024, FAKE, None) == -1


def test_multi_query_plan_and_limits(lib):
    """T query rows per sequence multiply the rows of each KV group: g * T picks the flavour and
    the head tile (g = 2, T = 2 -> 4 rows and g = 1, T = 3 -> 3 rows on the matrix cores; g = 1,
    T = 2 -> vector ALUs), the workspace grows with the units, and the fused append refuses
    T > 1."""
    assert _plan(lib, _desc(h_q=4, h_kv=2, n_queries=2), 100)[2] == 4
    assert _plan(lib, _desc(h_q=2, h_kv=2, n_queries=3), 100)[2] == 3
    assert _plan(lib, _desc(h_q=2, h_kv=2, n_queries=2), 100)[2] == 2
    assert _plan(lib, _desc(h_q=32, h_kv=8, n_queries=4), 100)[2] == 16
    assert _plan(lib, _desc(h_q=32, h_kv=1, n_queries=8), 100)[2] == 32  # 256 rows: 8 tiles of 32


def test_plan_caps_the_32_slot_register_ring_at_one_workgroup_per_cu(lib):
    # host-only: with no device the plan assumes 256 CUs; bf16 with 32 slots (MQA, g = 32) gets
    # one workgroup per CU, 16 slots and the 8-bit stages two
    mqa = _desc(batch=4, h_q=32, h_kv=1, cap=131072)
    assert _plan(lib, mqa, 131072)[1:] == (256, 32)
    assert _plan(lib, _desc(batch=16, h_q=32, h_kv=8, cap=32768), 32768)[1:] == (512, 4)
    fp8 = _desc(batch=4, h_q=32, h_kv=1, cap=131072, kv_dtype=2)
    assert _plan(lib, fp8, 131072)[1:] == (512, 32)


def test_plan_gives_one_workgroup_per_unit_when_the_vector_alu_units_match_the_cus(lib):
    # host-only (256 CUs assumed): MHA 8 x 32 heads = 256 units on the vector ALUs -> 256
    # workgroups, one whole unit each; 255 units keep the default two per CU, and so do the
    # 256 units of an 8-bit matrix-core workload
    assert _plan(lib, _desc(batch=8, h_q=32, h_kv=32, cap=4096), 4096)[:2] == (4096, 256)
    assert _plan(lib, _desc(batch=5, h_q=51, h_kv=51, cap=4096), 4096)[1] == 512
    assert _plan(lib, _desc(batch=32, h_q=64, h_kv=8, cap=16384, kv_dtype=2), 16384)[1] == 512
    one = _ws_size(lib, _desc(h_q=32, h_kv=8), 1000)[1]
    four = _ws_size(lib, _desc(h_q=32, h_kv=8, n_queries=4), 1000)[1]
    assert four > one > 0
    d = _desc(n_queries=2)
    rc, n = _ws_size(lib, d, 100)
    assert lib.decode_attn_append_run(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, None, FAKE, FAKE,
                                      n, None) == -2
    assert lib.decode_attn_append_combine(ctypes.byref(d), FAKE, 100, FAKE, FAKE, n, None) == -2


def test_static_entry_rejects_work_beyond_its_scratch(lib):
    """decode_attn_run_static holds its partials in a 16 MiB static scratch: a plan that needs
    more is refused on the host (DA_ERR_WORKSPACE) before anything is launched."""
    big = _desc(batch=1024, h_q=32, h_kv=32, cap=4096)
    rc, n = _ws_size(lib, big, 4096)
    assert rc == 0 and n > (16 << 20) - (256 << 10)
    assert lib.decode_attn_run_static(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, 4096, None, FAKE, None, None) == -3
    assert b"static scratch" in lib.da_last_error()
    d = _desc()
    assert lib.decode_attn_run_static(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 100, None, None, None, None) == -1
    assert lib.decode_attn_run_static(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 100, None, FAKE,
                                      ctypes.c_void_p(0x10002), None) == -1


@pytest.mark.parametrize("kw,max_len,ok", [
    (dict(q_dtype=0, kv_dtype=0), 8 << 20, False),       # fp32 d=128: 512-byte rows, 4 GiB
    (dict(q_dtype=0, kv_dtype=0), (8 << 20) - 4096, True),
    (dict(), 16 << 20, False),                            # bf16 d=128: 256-byte rows
    (dict(), (16 << 20) - 8192, True),
    (dict(kv_dtype=2, d_k=64, d_v=64), 64 << 20, False),  # fp8 d=64: 64-byte rows
])
def test_slots_beyond_32_bit_offsets_are_refused(lib, kw, max_len, ok):
    """The kernels' buffer offsets within one (sequence, KV head) slot are 32-bit: a max_len
    whose rows span 4 GiB or more is refused on the host (DA_ERR_UNSUPPORTED) instead of
    wrapping on the device."""
    d = _desc(cap=max_len, batch=1, h_q=2, h_kv=1, **kw)
    rc, _ = _ws_size(lib, d, max_len)
    assert rc == (0 if ok else -2), lib.da_last_error()


def test_single_pass_choice(lib):
    """The one-call entry points take the single pass when every sequence's K and V bytes at
    max_len are at most 1 MiB, unless a path or block_rows is given; da_plan then reports its
    workgroups (every unit cut into ceil(max_len / 64) splits, at most 64) and the vector-ALU
    head tile."""
    one = _desc(batch=1, h_q=1, h_kv=1, d_k=64, d_v=64, cap=1024, q_dtype=0, kv_dtype=0, path=0)
    assert _plan(lib, one, 1024) == (64, 16, 1)              # fp32 d=64: 512 KiB per sequence
    gqa = _desc(batch=16, h_q=32, h_kv=8, cap=32768, path=0)
    assert _plan(lib, gqa, 256) == (64, 16 * 8 * 4, 4)       # 8 KV heads x 256 rows x 512 B = 1 MiB
    assert _plan(lib, gqa, 257)[1] == -(-16 * 8 * 257 // 256)   # beyond: the split path, 256-row shares
    assert _plan(lib, _desc(batch=16, h_q=32, h_kv=8, cap=32768, path=2), 32768) == (512, 16 * 8 * 64, 4)
    assert _plan(lib, _desc(batch=16, h_q=32, h_kv=8, cap=32768, path=0, block_rows=64), 200)[1] > 16
    assert _ws_size(lib, _desc(path=2, block_rows=64), 100)[0] == -1
    assert _ws_size(lib, _desc(path=3), 100)[0] == -1
    # the single pass runs on the vector ALUs: the matrix-core flavour refuses it, the automatic
    # flavour falls back to the split path
    rc = lib.da_plan(ctypes.byref(_desc(path=2, flavour=2)), 100, None, None, None, None)
    assert rc == -2
    pa = ctypes.c_int32(-1)
    assert lib.da_plan(ctypes.byref(one), 1024, None, None, None, ctypes.byref(pa)) == 0 and pa.value == 2
    assert lib.da_plan(ctypes.byref(gqa), 4096, None, None, None, ctypes.byref(pa)) == 0 and pa.value == 1
    # the workspace does not depend on the path
    assert _ws_size(lib, _desc(path=0), 100) == _ws_size(lib, _desc(path=1), 100)


def test_shard_entry_points_validate_on_the_host(lib):
    """decode_attn_run_lse needs out and a 4-byte aligned lse and takes decode_attn_run's
    workspace; decode_attn_merge_lse checks its sizes and pointers before launching, and
    merges zero rows without launching anything."""
    d = _desc()
    rc, n = _ws_size(lib, d, 1000)
    assert rc == 0
    args = (ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 1000, None)
    assert lib.decode_attn_run_lse(*args, None, FAKE, FAKE, n, None) == -1
    assert lib.decode_attn_run_lse(*args, FAKE, None, FAKE, n, None) == -1
    assert lib.decode_attn_run_lse(*args, FAKE, ctypes.c_void_p(0x10002), FAKE, n, None) == -1
    assert lib.decode_attn_run_lse(*args, FAKE, FAKE, FAKE, n - 1, None) == -3
    merge = lib.decode_attn_merge_lse
    assert merge(0, 128, 4, None, None, None, None, None) == 0  # nothing to merge
    for rows, dd, shards in [(-1, 128, 2), (10, 6, 2), (10, 0, 2), (10, 8192, 2), (10, 128, 0), (10, 128, 5000)]:
        assert merge(rows, dd, shards, FAKE, FAKE, FAKE, None, None) == -1, (rows, dd, shards)
    assert merge(10, 128, 2, None, FAKE, FAKE, None, None) == -1
    assert merge(10, 128, 2, ctypes.c_void_p(0x10004), FAKE, FAKE, None, None) == -1  # outs misaligned
    assert merge(10, 128, 2, FAKE, ctypes.c_void_p(0x10002), FAKE, None, None) == -1  # lses misaligned
    assert merge(10, 128, 2, FAKE, FAKE, FAKE, ctypes.c_void_p(0x10001), None) == -1  # lse misaligned


C_PROGRAM = r"""
#include "decode_attn.h"
#include <stdio.h>
#include <string.h>

int main(void) {
    /* the grouped-query workload's descriptor, built from C */
    da_desc d;
    memset(&d, 0, sizeof d);
    d.batch = 16; d.h_q = 32; d.h_kv = 8; d.d_k = 128; d.d_v = 128; d.cap = 32768;
    d.q_dtype = DA_BF16; d.kv_dtype = DA_BF16; d.scale = 0.08838834764f; d.path = DA_PATH_SPLIT;
    size_t bytes = 0;
    int rc = da_workspace_size(&d, 32768, &bytes);
    int32_t rows = 0, blocks = 0, heads = 0, path = 0;
    int rc2 = da_plan(&d, 32768, &rows, &blocks, &heads, &path);
    /* host-side refusals, nothing launched */
    int rc3 = decode_attn_run(&d, NULL, NULL, NULL, NULL, 100, NULL, NULL, NULL, 0, NULL);
    int rc4 = decode_attn_merge_lse(0, 128, 2, NULL, NULL, NULL, NULL, NULL);
    printf("%d %zu %d %d %d %d %d %s\n", rc, bytes, rc2, heads, path, rc3, rc4, da_status_string(rc3));
    return 0;
}
"""


def test_header_is_plain_c_and_links(tmp_path, lib):
    """include/decode_attn.h compiles as C99 and a C program links against the library and
    calls its host-side entry points (plan, workspace size, argument refusal) with no GPU."""
    import shutil
    import subprocess
    if not shutil.which("gcc"):
        pytest.skip("gcc is not available")
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(_lib.library_path())
    inc = os.path.dirname(HEADER)
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", f"-I{inc}", str(src), "-o", str(exe),
                           f"-L{libdir}", "-ldecode_attn", f"-Wl,-rpath,{libdir}"])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    rc, nbytes, rc2, heads, path, rc3, rc4, status = out.stdout.split(maxsplit=7)
    assert (int(rc), int(rc2), int(heads), int(path), int(rc3), int(rc4)) == (0, 0, 4, 1, -1, 0)
    assert int(nbytes) > 0 and status.strip() == "invalid argument"
