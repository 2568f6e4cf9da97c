"""The C ABI's host code (argument checks, object lifetimes, registration bookkeeping,
launch planning) built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer
and driven through every entry point, with the HIP runtime and the kernel launchers
replaced by host stand-ins (tests/sanitize/).  No GPU: the kernels are not run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")


def test_abi_host_code_under_asan_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if not gxx or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path / "abi_sanitized")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROOT, 'rank_adapter_gemm_build_amd', 'csrc')}",
           os.path.join(ROOT, "rank_adapter_gemm_build_amd", "csrc", "api.cpp"), os.path.join(HERE, "hip_stubs.cpp"),
           os.path.join(HERE, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               RAXLORA_LOG="1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    assert "0 failures" in r.stdout
    # RAXLORA_LOG: one line per launch, naming the path the plan chose
    log = [l for l in r.stderr.splitlines() if l.startswith("raxlora: ")]
    assert any("mode=slot" in l for l in log) and any("mode=tiles" in l for l in log), r.stderr[-2000:]
    assert any(l.startswith("raxlora: grouped shrink") for l in log)
