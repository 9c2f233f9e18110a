"""Builds the gfx950 HIP library libnvfp4moe.so in-tree (package directory),
and its debug twin libnvfp4moe_debug.so (NVFP4_DEBUG_CHECKS: the routing
kernels check the data preconditions on the device and report them in the
workspace's precondition word; only the sources that read the flag are
compiled twice).

Every kernel is compiled for gfx950 only, with -ffp-contract=off and correctly
rounded fp32 division (the quantizer's bit-exact contract), and with packed
FP32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libnvfp4moe.so")
DEBUG_LIB = os.path.join(HERE, "libnvfp4moe_debug.so")
SOURCES = ["quantize.hip", "route.hip", "gemm.hip", "single_pass.hip", "backward.hip",
           "combine.hip", "capi.hip", "noalloc.hip"]
DEBUG_SOURCES = ["route.hip", "capi.hip"]      # the sources that read NVFP4_DEBUG_CHECKS

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str, verbose: bool, debug: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, ("debug_" if debug else "") + src.replace(".hip", ".o"))
    extra = ["-DNVFP4_DEBUG_CHECKS"] if debug else []
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature flag: drop that note
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    units = [(s, False) for s in SOURCES] + [(s, True) for s in DEBUG_SOURCES]
    jobs = min(len(units), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda u: _compile(u[0], verbose, u[1]), units))
    release = objs[:len(SOURCES)]
    debug_objs = dict(zip(DEBUG_SOURCES, objs[len(SOURCES):]))
    _link(release, LIB, verbose)
    _link([debug_objs.get(s, o) for s, o in zip(SOURCES, release)], DEBUG_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
