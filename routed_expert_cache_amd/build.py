"""Build the HIP library in-tree: hipcc for gfx950 -> libmoe_gfx950.so.

    python -m routed_expert_cache_amd.build

Every source is compiled on each call (the build is the "does it build"
check); objects go to routed_expert_cache_amd/_build/.  The device assembly
of every source is then checked for registers of hand-timed asm loads that
the compiler touches before their wait (asm_check.py); the build fails on
any.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from routed_expert_cache_amd import asm_check

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_gfx950.so")
SOURCES = ["route_topk.hip", "cache.hip", "forward.hip", "host_signal.hip", "host_exec.cpp"]
GPU_SOURCES = [s for s in SOURCES if s.endswith(".hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # packed FP32 arithmetic stays off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-x", "c++", "-I" + os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "include"),
              "-D__HIP_PLATFORM_AMD__", "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    # host-only C++ (the CPU executor) is compiled as plain C++ against the HIP runtime headers
    flags = FLAGS if src.endswith(".hip") else HOST_FLAGS
    cmd = [HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    return obj, warn


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
        list(ex.map(lambda s: asm_check.check_sources(CSRC, [s], HIPCC, FLAGS), GPU_SOURCES))
    for obj, warn in results:
        if warn.strip() and verbose:
            print(warn, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
