"""The C-ABI layer (argument checks, size arithmetic, workspace carving) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, its kernel launchers replaced by host stubs
(tests/host_sanitize/), and run over every entry point on the CPU.  Any sanitizer finding or
unmet expectation fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_c_abi_layer_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "dsa_abi_harness")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "sparse_attention_long_gemm_amd", "csrc"), "-I" + HERE,
           os.path.join(ROOT, "sparse_attention_long_gemm_amd", "csrc", "dsa_api.cpp"),
           os.path.join(HERE, "stub_launchers.cpp"), os.path.join(HERE, "harness.cpp"),
           "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr[-4000:]
