"""The C ABI's host-side logic (argument checks, size queries, work plans, the page-table and
shared-prefix checks) built for the host with AddressSanitizer and UndefinedBehaviorSanitizer and
driven through extreme and invalid arguments (tests/sanitize/abi_checks.cpp; the kernels' launch
functions are stubs, so nothing reaches a GPU).  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_host_abi_logic_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("needs g++ and the HIP runtime library")
    exe = tmp_path / "abi_checks"
    cmd = [gxx, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "bit_rotated_kv_decode_amd", "csrc"),
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-g", "-O1",
           os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp"),
           os.path.join(ROOT, "bit_rotated_kv_decode_amd", "csrc", "oscar_api.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "all expectations hold" in out
