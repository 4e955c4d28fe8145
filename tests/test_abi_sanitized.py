"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/helpers/abi_sanitize.cpp links the library's host code (argument checks,
workspace layout) with stub kernel launchers and calls every entry point with
bad arguments and workspace sizing with extreme parameters; the sanitizers are
applied to host code only.  No GPU is involved.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_api_under_asan_and_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_sanitize")
    cmd = [hipcc, "-std=c++17", "-O1", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "long_context_sparse_approx_amd", "csrc"),
           os.path.join(ROOT, "tests", "helpers", "abi_sanitize.cpp"),
           os.path.join(ROOT, "long_context_sparse_approx_amd", "csrc", "ssa_api.cpp"),
           "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-2000:]
    assert run.stdout.strip().endswith("ok")
