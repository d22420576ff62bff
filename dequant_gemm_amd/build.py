"""Build libcubic.so (gfx950) in-tree with hipcc.

    python -m dequant_gemm_amd.build          # compile every source, link the library

Objects go to dequant_gemm_amd/_build/, the library to dequant_gemm_amd/lib/.
Every call compiles all sources (no staleness heuristics).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libcubic.so")
SOURCES = ["basic.hip", "fit.hip", "gemv.hip", "gemv_rows.hip", "moe.hip", "moe_a8.hip", "tiled.hip", "prefill.hip", "prefill_a8.hip", "skinny.hip", "api.cpp"]
ARCH = os.environ.get("CUBIC_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# Packed-fp32 instructions are disabled for device code; hipcc's host pass warns
# that it does not know the feature, which is harmless.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# The group fitter takes finite weights only (its C-ABI says so): without NaN
# semantics the first operand of its running minimum needs no canonicalising
# max, one VALU instruction in thirteen of its inner loop.
SOURCE_FLAGS = {"fit.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2) // 2), 8)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_floors(verbose)
    return LIB


FLOORS_LIB = os.path.join(LIBDIR, "libcubic_floors.so")


def build_floors(verbose: bool = True) -> str:
    """The benchmark's floor kernels (csrc/floors.hip) as a library of their own."""
    obj = _compile("floors.hip")
    tmp = FLOORS_LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", obj, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, FLOORS_LIB)
    if verbose:
        print(f"built {FLOORS_LIB}")
    return FLOORS_LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
