"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, run
on the CPU: the oracle (oracle/mxoracle.c, built with gcc, serial) under
tests/sanitize/oracle_driver.c, and the library's host side (argument
validation and size helpers) under tests/sanitize/api_driver.cpp, built with
hipcc with the sanitizers on the host pass only.  The API driver makes no
call that reaches a launch, and runs only where no GPU is present, with HIP
shown no device."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "tests", "_build")
CSRC = os.path.join(ROOT, "fp8_precision_quantization_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, **kw)


def test_oracle_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_asan")
    b = _run(["gcc", "-std=c99", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-Wall", "-Werror", "-Wno-unknown-pragmas",
              os.path.join(ROOT, "oracle", "mxoracle.c"), os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    assert b.returncode == 0, b.stderr
    r = _run([exe], env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr
    assert "oracle sanitizer run clean" in r.stdout


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present; this build runs where none is")
def test_library_host_code_under_asan_ubsan():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "api_asan")
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    b = _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, os.path.join(HERE, "api_driver.cpp"),
              "-o", exe])
    assert b.returncode == 0, b.stderr[-4000:]
    r = _run([exe], env=ENV, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "api sanitizer run clean" in r.stdout
