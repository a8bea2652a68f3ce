"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

tests/native/host_api_asan.cpp compiles the ABI layer (argument validation, workspace carving,
launch sequencing) with the system C++ compiler and sanitizers, and replaces the device launchers
by stubs that write exactly the bytes each kernel writes (and read the workspace extents it reads)
into host buffers of the sizes the workspace queries report.  Every call's validation and
carving runs for bf16 and fp32 problems; an undersized workspace or a mis-carved sub-buffer is a
heap-buffer-overflow, undefined behaviour aborts, and each status code is checked."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "host_api_asan.cpp")
ROCM = "/opt/rocm"


def test_host_api_under_address_and_ub_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("needs g++ and the HIP runtime library")
    exe = tmp_path / "host_api_asan"
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", SRC, "-o", str(exe),
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr + r.stdout).lower() and "cannot find" in r.stderr:
        pytest.skip("the compiler has no sanitizer runtime")
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("DSV_DEBUG_VALIDATE", None)
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    out = run.stdout + run.stderr
    assert run.returncode == 0 and "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "host API checks passed" in out
