"""Build libkda.so in-tree with hipcc for gfx950 (no GPU needed to compile).

    python -m channel_gated_delta_amd.build

Each translation unit under csrc/ compiles in parallel; the shared object exports
only the C ABI declared in include/kda.h (hidden visibility elsewhere).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkda.so")
ARCH = "gfx950"

SOURCES = ["kda_api.cpp", "kda_scratch.hip", "kda_prologue.hip", "kda_decode.hip", "kda_chunk_bf16.hip",
           "kda_chunk_bf16_bf16out.hip", "kda_chunk_f32.hip", "kda_chunk_bf16_gz.hip",
           "kda_chunk_bf16_bf16out_gz.hip", "kda_chunk_f32_gz.hip", "kda_epilogue.hip",
           "kda_chunk_bf16_gdn.hip", "kda_chunk_bf16_bf16out_gdn.hip", "kda_chunk_f32_gdn.hip"]

# Packed-fp32 instructions are disabled for device code: hipcc -O3 would emit
# v_pk_{add,mul,fma}_f32 from plain float code otherwise.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden",
         "-Wall", "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-I" + INCLUDE, "-I" + CSRC]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: libkda needs ROCm's hipcc to build")
    return path


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc()] + FLAGS
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line.
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = True) -> str:
    """Compile every HIP source for gfx950 and link libkda.so next to this file."""
    with tempfile.TemporaryDirectory(prefix="kda_build_") as tmp:
        objs = [os.path.join(tmp, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
        workers = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(_compile, SOURCES, objs))
        out_tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", out_tmp] + objs
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stderr)
        os.replace(out_tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
