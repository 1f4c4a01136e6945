"""Checks on the gfx950 assembly of the kernel library (CPU only: hipcc cross-compiles).

The 8-bit segment issues its LDS DMA as inline assembly that writes M0 (`lds_dma16`). M0 is
a register the compiler reserves, so it does not save or restore it around the statement:
the code is correct only while nothing else in the device code keeps a value in M0. This
test compiles the library's device code to assembly and checks that every M0 access is
one of those statements' own `s_mov_b32 m0, sN`, inside its inline-assembly block and
followed by the DMA that reads it.
"""
import os
import re
import shutil
import subprocess

import pytest

from decode_attention_kv_split_amd import build

HIPCC = build.HIPCC


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc is not available")
    out = tmp_path_factory.mktemp("asm") / "decode_attn.s"
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", build.SRC, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text().splitlines()


def test_m0_is_only_written_by_the_lds_dma_statements(device_asm):
    lines = device_asm
    m0 = re.compile(r"\bm0\b")
    uses = [i for i, l in enumerate(lines) if m0.search(l.split(";")[0])]
    assert uses, "no LDS DMA statement found in the device code"
    for i in uses:
        code = lines[i].split(";")[0].strip()
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", code), f"M0 used outside the LDS DMA statement: {code!r}"
        block = [l.strip() for l in lines[i - 2:i + 4]]
        assert block[0] == ";;#ASMSTART" and block[1] == "s_nop 4", block
        assert block[3] == "s_nop 0" and re.fullmatch(r"buffer_load_dwordx4 v\d+, s\[\d+:\d+\], 0 offen nt lds", block[4]), block
        assert block[5] == ";;#ASMEND", block
