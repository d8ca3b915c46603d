"""Build libfp8q.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m fp8_fine_grained_online_amd.build [--verbose]
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libfp8q.so")

SOURCES = ["quant.hip", "retile.hip", "norm.hip", "moe.hip", "gemm.hip", "gemm_qa.hip", "api.cpp"]
HEADERS = ["common.hpp", "tiles.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
    # packed-FP32 VALU forms are disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no implicit multiply-add fusion: every rounding the kernels' arithmetic
    # is specified with happens as written (HIP's header versions of the
    # __fmul_rn/__dmul_rn intrinsics are plain products that would otherwise
    # be contracted into a following addition); FMAs are always explicit
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    build_probes(verbose)
    return LIB_PATH


# Test-only GPU probes (tests/probes/*.hip), each built into its own shared
# library next to its source; the product library never loads them.
PROBE_DIR = os.path.join(ROOT, "tests", "probes")


def build_probes(verbose: bool = False):
    if not os.path.isdir(PROBE_DIR):
        return []
    out = []
    for src in sorted(f for f in os.listdir(PROBE_DIR) if f.endswith(".hip")):
        lib = os.path.join(PROBE_DIR, "lib" + src[:-4] + ".so")
        _run([HIPCC, *FLAGS, "-shared", "-x", "hip", os.path.join(PROBE_DIR, src), "-o", lib + ".tmp"],
             verbose)
        os.replace(lib + ".tmp", lib)
        out.append(lib)
    return out


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
