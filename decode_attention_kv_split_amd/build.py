"""Build the gfx950 HIP library in-tree: libdecode_attn.so next to this file.

One translation unit (csrc/decode_attn.hip) holds the kernels and the C ABI
declared in include/decode_attn.h. Flags:
  --offload-arch=gfx950                 MI355X (CDNA4) only
  -fno-gpu-flush-denormals-to-zero      fp32 subnormals kept (the fp8 decoder relies on them)
  -target-feature -packed-fp32-ops      no packed fp32 VALU instructions are generated
  -amdgpu-mfma-vgpr-form=1              matrix-core accumulators in ordinary VGPRs: the 32-head
                                        kernel (one wave per SIMD) otherwise keeps its output
                                        tile in accumulation registers and copies it to and
                                        from VGPRs around every tile (MQA 46.2 -> 44.9 us)
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "decode_attn.hip")
HEADER = os.path.join(ROOT, "include", "decode_attn.h")
LIB = os.path.join(PKG, "libdecode_attn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
         "-fno-gpu-flush-denormals-to-zero",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-I", os.path.join(ROOT, "include")]


def _code_tokens(text: str) -> str:
    """The source without comments, whitespace runs collapsed (string and character literals
    kept as written), so that edits of comments or layout leave the digest alone."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def code_digest() -> str:
    """sha256 of the kernel source and header (comments and layout aside) and the compiler
    flags (repository paths made relative): it names the device code that a measurement was
    taken on."""
    import hashlib
    parts = [_code_tokens(open(p, encoding="utf-8").read()) for p in (SRC, HEADER)]
    flags = [os.path.relpath(f, ROOT) if f.startswith(ROOT) else f for f in FLAGS]
    return hashlib.sha256("\0".join(parts + [" ".join(flags)]).encode()).hexdigest()


def build_library(verbose: bool = False) -> str:
    """Compile the HIP library (always recompiles) and return its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
