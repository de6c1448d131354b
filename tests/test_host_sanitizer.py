"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

fa_api.cpp (every argument check, the parameter structs handed to the
launchers, the workspace arithmetic, the thread-local error string) is built
host-only with g++ -fsanitize=address,undefined against stub launchers
(tests/sanitizer/stubs.cpp) and driven by tests/sanitizer/abi_driver.cpp:
refusals of bad arguments, valid calls of every entry point through to the
stubs, workspace bounds, size products past 32 bits, and two threads failing
at once. No GPU and no HIP runtime are involved; the kernels are not built.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INCLUDE), reason="needs g++ and HIP headers")
def test_c_abi_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "abi_asan"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "io_aware_flashattention_amd", "csrc"),
           os.path.join(ROOT, "io_aware_flashattention_amd", "csrc", "fa_api.cpp"),
           os.path.join(ROOT, "tests", "sanitizer", "stubs.cpp"),
           os.path.join(ROOT, "tests", "sanitizer", "abi_driver.cpp"), "-o", str(exe), "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "ALL OK" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
