"""Build libhsla.so and libhsla_debug.so for gfx950 with hipcc (in-tree,
next to this file).  The debug library is the same code with
HSLA_DEBUG_CHECKS defined in the C ABI layer: every entry point checks the
lengths and block tables its kernels will use before it launches them.

    python hybrid_sparse_linear_block_amd/build.py

(run by path: importing the package first would load the library that is
being rebuilt).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libhsla.so")
DEBUG_LIB = os.path.join(HERE, "libhsla_debug.so")
SOURCES = ["hsla_api.cpp", "decode.hip", "build.hip", "append.hip", "check.hip"]
DEBUG_DEFINES = ["-DHSLA_DEBUG_CHECKS=1"]
ARCH = os.environ.get("HSLA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++20",
    # packed fp32 VALU forms stay disabled on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no wavefront-level rewrite of atomics: it reads an atomic's result back
    # at once, which would drain the attention loop's loads at every claim
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(job) -> str:
    src, debug = job
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ("_debug" if debug else "") + ".o")
    cmd = [HIPCC, *CFLAGS, *(DEBUG_DEFINES if debug else []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    """Both libraries: the kernels are compiled once; only the C ABI layer
    differs (HSLA_DEBUG_CHECKS)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + [("hsla_api.cpp", True)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(_compile, jobs))
    release, api_debug = objs[:len(SOURCES)], objs[len(SOURCES)]
    _link(release, LIB)
    _link([api_debug] + release[1:], DEBUG_LIB)
    if verbose:
        print(f"built {LIB} and {DEBUG_LIB}")
    return LIB


if __name__ == "__main__":
    build()
