"""The C ABI's host code (gdn_api.hip: validation, workspace carving and
dispatch) built with AddressSanitizer and UndefinedBehaviorSanitizer on the
host and run without a GPU: tests/sanitize/launch_stubs.cpp stands in for the
kernel launchers and checks every device pointer they receive against the
caller's regions (tensors and workspace), and tests/sanitize/api_driver.cpp
calls every entry point over a grid of problems, valid and invalid."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_deltanet_recurrence_frame_amd", "csrc")
INC = os.path.join(ROOT, "include")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="ROCm compilers not found")
def test_api_host_code_under_asan_and_ubsan(tmp_path):
    d = str(tmp_path)
    # sanitizers on the host side only (-Xarch_host before each); the API's
    # device code (its static scratch) is built for gfx950 as in the library
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    common = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-I", INC, "-I", CSRC,
              "-I", SAN]
    _run([HIPCC, "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-Wno-unused-command-line-argument"] + common + san +
         ["-c", os.path.join(CSRC, "gdn_api.hip"), "-o", "api.o"], d)
    _run([HIPCC, "-x", "hip", "--cuda-host-only", "-Wno-unused-command-line-argument"] + common +
         san + ["-c", os.path.join(SAN, "launch_stubs.cpp"), "-o", "stubs.o"], d)
    _run([CLANG, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"] + common +
         ["-c", os.path.join(SAN, "api_driver.cpp"), "-o", "driver.o"], d)
    _run([CLANG, "-fsanitize=address,undefined", "api.o", "stubs.o", "driver.o",
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", "driver"], d)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([os.path.join(d, "driver")], cwd=d, capture_output=True, text=True,
                       env=env, timeout=300)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-5000:]
    assert "0 failed" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
