"""The library's host code under AddressSanitizer and UndefinedBehavior-
Sanitizer, on the CPU (no GPU, no HIP runtime).

api.cpp (argument checks, workspace sizing, the band and selection-group
schedule) and plan.cpp (selection-path choice, fused-handoff layout, key
splits) are compiled as plain host C++ by the ROCm clang++ (it knows
_Float16 on x86-64) together with host stubs of the HIP runtime and
of every kernel launcher (tests/sanitize/hip_stubs.cpp). A seeded fuzz
(tests/sanitize/fuzz_main.cpp) then drives every entry point with thousands
of descriptors, valid and broken: zero and one query, band edges, the largest
top-k and compressed-row counts, positions near the int32 limit. The stubs
check that every launch a call makes stays inside the arrays the C ABI
documents for that descriptor (and the workspace it asked for); the
sanitizers abort on any memory error, signed overflow, or division by zero.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_long_context_int8_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")


@pytest.fixture(scope="module")
def fuzz_bin(tmp_path_factory):
    gxx = next((c for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")) if c and os.path.exists(c)),
               None)
    if gxx is None:
        pytest.skip("clang++ not available")
    hip_inc = "/opt/rocm/include"
    if not os.path.isdir(os.path.join(hip_inc, "hip")):
        pytest.skip("HIP headers not available")
    out = str(tmp_path_factory.mktemp("sanitize") / "fuzz")
    cmd = [gxx, "-x", "c++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", hip_inc, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", SAN,
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(SAN, "hip_stubs.cpp"), os.path.join(SAN, "fuzz_main.cpp"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_host_code_fuzz_under_sanitizers(fuzz_bin, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([fuzz_bin, "4000", str(seed)], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "fuzz: 4000 cases" in res.stdout
