"""The C ABI's host code (fa2_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/abi_host_check.cpp links fa2_api.cpp against stub kernel launchers (no GPU code is built
or run) and calls every entry point with invalid and valid arguments, checking the status codes
and the argument blocks the launchers receive. It is compiled here with g++ (host code only),
-fsanitize=address,undefined and no recovery, so any out-of-bounds access, use of freed memory,
leak or undefined behaviour in the validation and marshalling code fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "exact_io_aware_42_amd")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_abi_host_code_under_sanitizers():
    out_dir = os.path.join(PKG, "_build", "sanitize")
    os.makedirs(out_dir, exist_ok=True)
    exe = os.path.join(out_dir, "abi_host_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}",
           f"-I{os.path.join(PKG, 'csrc')}", os.path.join(PKG, "csrc", "fa2_api.cpp"),
           os.path.join(ROOT, "tests", "abi_host_check.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(run.stdout, run.stderr)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "abi host checks ok" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
