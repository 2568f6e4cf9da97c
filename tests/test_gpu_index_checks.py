"""The index-checking build of the library (libraxlora_debug.so, compiled with
-DRAXLORA_DEBUG: every index a kernel takes from memory -- token ids, slots, sorted
positions, workspace rows -- checked against its range, a failed check counted and
its access sent to index 0) under a set of the GPU parity tests.  They run in a child
process that loads that build instead of the release one (RAXLORA_LIBRARY); there
every test must pass and leave no failed check (tests/conftest.py)."""
import os
import subprocess
import sys

import pytest

from rank_adapter_gemm_build_amd import build as B

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEBUG_LIB = os.path.join(ROOT, "rank_adapter_gemm_build_amd", "libraxlora_debug.so")
FILES = ["tests/test_gpu_slot_mode.py", "tests/test_gpu_route_linear.py", "tests/test_gpu_group.py",
         "tests/test_gpu_parity.py", "tests/test_gpu_fp8.py", "tests/test_gpu_embedding.py"]


@pytest.mark.timeout(900)
def test_parity_suites_on_the_index_checking_build():
    assert os.path.exists(DEBUG_LIB), \
        f"{DEBUG_LIB} is missing: build it with `python rank_adapter_gemm_build_amd/build.py --debug`"
    # the sources it was linked from (recorded by the build), compared by content
    with open(B.digest_path(DEBUG_LIB)) as fh:
        built = fh.read().strip()
    assert built == B.source_digest(), \
        f"{DEBUG_LIB} was built from other sources: rebuild it with `python rank_adapter_gemm_build_amd/build.py --debug`"
    env = dict(os.environ, RAXLORA_LIBRARY=DEBUG_LIB, RAXLORA_EXPECT_INDEX_CHECKS="1")
    cmd = [sys.executable, "-u", "-m", "pytest", *FILES, "-m", "gpu", "-x", "-q", "-p", "no:cacheprovider",
           "--timeout", "300", "--timeout-method", "thread"]
    print("index-checking build:", " ".join(cmd[3:]), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=840)
    tail = "\n".join((r.stdout + r.stderr).splitlines()[-25:])
    print(tail, flush=True)
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and " failed" not in r.stdout, tail
