"""Build the HIP library (libraxlora.so) for gfx950, in-tree.

Every source under csrc/ is compiled with hipcc for gfx950 (one object per file, in
parallel) and linked into ``rank_adapter_gemm_build_amd/libraxlora.so``.  All HIP code
is compiled with the packed-fp32 feature turned off, so hipcc never emits packed fp32
arithmetic.

    python -m rank_adapter_gemm_build_amd.build          # or: python rank_adapter_gemm_build_amd/build.py
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libraxlora.so")
# the index-checking variant (-DRAXLORA_DEBUG): the same kernels with every index taken
# from memory checked against its range (lora_index_checks)
BUILD_DEBUG = os.path.join(ROOT, "_build_debug")
LIB_DEBUG = os.path.join(PKG, "libraxlora_debug.so")

ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
HIP_ONLY = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-munsafe-fp-atomics"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def source_digest() -> str:
    """sha256 (first 16 hex digits) of every file under csrc/ and include/, names and
    contents: what a built library was compiled from, independent of file times."""
    h = hashlib.sha256()
    for d in (CSRC, INCLUDE):
        for f in sorted(os.listdir(d)):
            path = os.path.join(d, f)
            if os.path.isfile(path):
                with open(path, "rb") as fh:
                    h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def digest_path(lib: str) -> str:
    """The file beside a built library that records source_digest() at link time."""
    return lib + ".sources"


def _compile(src: str, extra, build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc(), "-x", "hip", *HIP_ONLY, *COMMON, *extra, "-c", src, "-o", obj]
    else:  # host-only C++: no device pass
        cmd = [hipcc(), *COMMON, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l and "ignoring feature" not in l)
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def _stale(src: str, headers, build_dir: str = BUILD) -> bool:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(f) > t for f in [src, *headers])


def build(verbose: bool = True, extra=(), incremental: bool = False, debug: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library; returns its path.
    incremental: recompile only sources older than themselves or any header.
    debug: the index-checking variant, libraxlora_debug.so, from objects of its own."""
    build_dir, lib = (BUILD_DEBUG, LIB_DEBUG) if debug else (BUILD, LIB)
    extra = list(extra) + (["-DRAXLORA_DEBUG"] if debug else [])
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    headers = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")] + \
        [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]
    todo = [s for s in srcs if not incremental or _stale(s, headers, build_dir)]
    with cf.ThreadPoolExecutor(max_workers=max(1, min(8, len(todo)))) as ex:
        list(ex.map(lambda s: _compile(s, extra, build_dir), todo))
    objs = [os.path.join(build_dir, os.path.basename(s) + ".o") for s in srcs]
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    with open(digest_path(lib), "w") as fh:
        fh.write(source_digest() + "\n")
    if verbose:
        print(f"built {lib} from {len(srcs)} sources for {ARCH}")
    return lib


if __name__ == "__main__":
    build(incremental="--incremental" in sys.argv[1:], debug="--debug" in sys.argv[1:])
