"""The built library's matrix products never write a destination that partially
overlaps their accumulator input.

A 16x16 MFMA with D = A B + C may accumulate in place (D and C the same four
registers) or into registers disjoint from C.  The compiler can also give D a
range shifted by half a tile against C (D two registers below or above C), and
the matrix unit then does not form the right sum: it writes part of D before it
has read the part of C that shares those registers.  The kernels keep such
products out by construction (``mma_sep`` and zero-accumulator products); this
test disassembles every gfx950 code object in libkda.so and checks the rule on
each MFMA, so that a later change or compiler cannot bring the overlap back
unnoticed.  Runs on the CPU.
"""
from __future__ import annotations

import os
import re
import shutil
import struct
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "channel_gated_delta_amd", "libkda.so")
LLVM_BIN = "/opt/rocm/llvm/bin"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

_RANGE = re.compile(r"^([va])\[(\d+):(\d+)\]$|^([va])(\d+)$")


def reg_range(tok: str):
    """('v'|'a', first, last) of a register operand, None for constants."""
    m = _RANGE.match(tok.strip())
    if not m:
        return None
    if m.group(1):
        return m.group(1), int(m.group(2)), int(m.group(3))
    return m.group(4), int(m.group(5)), int(m.group(5))


def partial_overlap(line: str) -> bool:
    """Whether an MFMA's destination overlaps its C operand without being it."""
    text = line.split("//")[0].strip()
    if not text.startswith("v_mfma"):
        return False
    ops = [o.strip() for o in text.split(None, 1)[1].split(",")]
    d, c = reg_range(ops[0]), reg_range(ops[3])
    if d is None or c is None or d[0] != c[0]:
        return False
    return d != c and not (d[2] < c[1] or c[2] < d[1])


def code_objects(fatbin: bytes):
    """The gfx950 code objects of a .hip_fatbin section (one offload bundle per
    translation unit, each a header of entries: offset, size, target id)."""
    out = []
    at = fatbin.find(BUNDLE_MAGIC)
    while at >= 0:
        n = struct.unpack_from("<Q", fatbin, at + 24)[0]
        p = at + 32
        for _ in range(n):
            off, size, idlen = struct.unpack_from("<QQQ", fatbin, p)
            p += 24
            tid = fatbin[p:p + idlen].decode()
            p += idlen
            if tid == TARGET and size:
                out.append(fatbin[at + off:at + off + size])
        at = fatbin.find(BUNDLE_MAGIC, at + 1)
    return out


def test_scanner_flags_half_tile_shifts():
    assert partial_overlap("v_mfma_f32_16x16x16_bf16 v[34:37], v[48:49], v[34:35], v[36:39]")
    assert partial_overlap("v_mfma_f32_16x16x16_bf16 v[20:23], v[6:7], v[36:37], v[18:21]")
    assert not partial_overlap("v_mfma_f32_16x16x32_bf16 v[84:87], v[38:41], v[84:87], v[84:87]")
    assert not partial_overlap("v_mfma_f32_16x16x32_bf16 v[36:39], v[84:87], v[34:37], v[80:83]")
    assert not partial_overlap("v_mfma_f32_16x16x32_bf16 v[84:87], v[38:41], v[84:87], 0")
    assert not partial_overlap("v_mfma_f32_16x16x4_f32 a[0:3], v1, v2, v[0:3]")


@pytest.mark.skipif(not os.path.exists(LIB), reason="libkda.so not built")
@pytest.mark.skipif(not os.path.exists(os.path.join(LLVM_BIN, "llvm-objdump")),
                    reason="ROCm llvm-objdump not installed")
def test_no_mfma_destination_half_overlaps_its_accumulator():
    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fatbin")
        subprocess.run([os.path.join(LLVM_BIN, "llvm-objcopy"), "--dump-section",
                        ".hip_fatbin=" + fat, LIB, os.path.join(tmp, "copy.so")],
                       check=True, capture_output=True)
        objs = code_objects(open(fat, "rb").read())
        assert len(objs) >= 10, "expected one gfx950 code object per HIP source"
        n_mfma, bad = 0, []
        for i, co in enumerate(objs):
            path = os.path.join(tmp, "co%d.o" % i)
            with open(path, "wb") as f:
                f.write(co)
            res = subprocess.run([os.path.join(LLVM_BIN, "llvm-objdump"), "-d", "--mcpu=gfx950",
                                  "--no-show-raw-insn", path],
                                 check=True, capture_output=True, text=True)
            for line in res.stdout.splitlines():
                if "v_mfma" in line:
                    n_mfma += 1
                    if partial_overlap(line.strip()):
                        bad.append(line.strip())
        assert n_mfma > 1000, "disassembly found too few MFMA instructions (%d)" % n_mfma
        assert not bad, "MFMA destination half-overlaps its accumulator:\n" + "\n".join(bad[:10])
