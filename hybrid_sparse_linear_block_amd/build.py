"""Build libhsla.so, libhsla_debug.so and libhsla_phases.so for gfx950 with
hipcc (in-tree, next to this file).  The debug library is the same code with
HSLA_DEBUG_CHECKS defined in the C ABI layer: every entry point checks the
lengths and block tables its kernels will use before it launches them.  The
phases library compiles the decode kernels with HSLA_PHASE_TIMESTAMPS: every
workgroup stamps its phases (a diagnostic build, read by bench.py --phases).

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
PHASES_LIB = os.path.join(HERE, "libhsla_phases.so")
SOURCES = ["hsla_api.cpp", "decode.hip", "build.hip", "append.hip", "check.hip"]
DEBUG_DEFINES = ["-DHSLA_DEBUG_CHECKS=1"]
PHASES_DEFINES = ["-DHSLA_PHASE_TIMESTAMPS=1"]
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
    src, variant = job   # variant: "", "debug" or "phases"
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + (f"_{variant}" if variant else "") + ".o")
    defines = {"": [], "debug": DEBUG_DEFINES, "phases": PHASES_DEFINES}[variant]
    cmd = [HIPCC, *CFLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
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
    """The three libraries: the release objects are compiled once; the debug
    library differs in its C ABI layer (HSLA_DEBUG_CHECKS), the phases
    library in its decode kernels (HSLA_PHASE_TIMESTAMPS)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = [(s, "") for s in SOURCES] + [("hsla_api.cpp", "debug"), ("decode.hip", "phases")]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(_compile, jobs))
    release, api_debug, decode_phases = objs[:len(SOURCES)], objs[len(SOURCES)], objs[len(SOURCES) + 1]
    assert SOURCES[0] == "hsla_api.cpp" and SOURCES[1] == "decode.hip"
    _link(release, LIB)
    _link([api_debug] + release[1:], DEBUG_LIB)
    _link([release[0], decode_phases] + release[2:], PHASES_LIB)
    if verbose:
        print(f"built {LIB}, {DEBUG_LIB} and {PHASES_LIB}")
    return LIB


if __name__ == "__main__":
    build()
