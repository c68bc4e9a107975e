"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The fp64 oracle (oracle/kda_oracle.c) linked with tests/sanitize/oracle_driver.c,
  which calls every oracle function on exact-size heap buffers: ragged and empty
  packed sequences, conv widths 1..4, history in place, special values, rejected
  arguments.
* The host half of libkda (channel_gated_delta_amd/csrc/kda_api.cpp: argument
  checks, status codes, launcher choice) linked with tests/sanitize/api_driver.cpp,
  whose stub launchers record what each entry point would launch; every entry
  point with valid arguments and with each class of invalid argument.

Both are built with gcc / g++ (host code only; nothing here touches a GPU), with
-fno-sanitize-recover so that any report fails the run.  A planted heap overflow
checks that the sanitizer build really catches one.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
HIP_INCLUDE = "/opt/rocm/include"


def build_and_run(cmd, exe, env_extra=None):
    res = subprocess.run(cmd + ["-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, "build failed:\n" + res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    env.update(env_extra or {})
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    r = build_and_run(["gcc", "-std=c99", "-fopenmp"] + SAN +
                      [os.path.join(ROOT, "oracle", "kda_oracle.c"),
                       os.path.join(HERE, "oracle_driver.c"), "-lm"],
                      str(tmp_path / "oracle_san"))
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INCLUDE),
                    reason="g++ or the HIP headers not available")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    csrc = os.path.join(ROOT, "channel_gated_delta_amd", "csrc")
    r = build_and_run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I" + HIP_INCLUDE,
                       "-I" + os.path.join(ROOT, "include"), "-I" + csrc] + SAN +
                      [os.path.join(csrc, "kda_api.cpp"), os.path.join(HERE, "api_driver.cpp")],
                      str(tmp_path / "api_san"))
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("body,report", [
    # one element past a heap block (ASan, or UBSan's object-size check, whichever fires first)
    ("volatile int *p = malloc(4 * sizeof(int)); p[argc + 3] = 1; free((void *)p);",
     ("heap-buffer-overflow", "insufficient space")),
    # signed overflow of a size computation, the bug class the ABI checks guard against
    ("volatile long long t = 9223372036854775807LL - 1 + argc; volatile long long u = t + 16;"
     " (void)u;", ("signed integer overflow",)),
], ids=["heap_overflow", "signed_overflow"])
def test_sanitizer_build_catches_planted_bugs(tmp_path, body, report):
    """The same flags on a planted bug must fail: the checks above are live."""
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\nint main(int argc, char **argv) { (void)argv; %s"
                   " return 0; }\n" % body)
    r = build_and_run(["gcc", "-std=c99"] + SAN + [str(src)], str(tmp_path / "planted"))
    assert r.returncode != 0 and any(m in r.stderr for m in report), r.stderr[-2000:]
