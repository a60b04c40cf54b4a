"""Build libqgemv.so (HIP for gfx950) in-tree with hipcc.

    python -m dequant_gemv_q4_amd.build            # build (always recompiles)
    python -m dequant_gemv_q4_amd.build --save-temps DIR   # also keep the gfx950 assembly

Each source compiles to an object in parallel (``_build/``), then one link.  Extra preprocessor
definitions for tuning sweeps can be passed with ``-D NAME=VALUE``.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqgemv.so")
BW_LIB = os.path.join(PKG, "libqgbw.so")       # the benchmark's bandwidth reference (bw_read.hip)
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["gemv_kernels.hip", "gemv_kernels_x.hip", "stream_kernels.hip", "stream_kernels_x.hip",
           "stream_kernels_g.hip",
           "mfma_kernels.hip", "gemm_kernels.hip", "abi.cpp"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed FP32 instructions stay off: the compiler must not form them from float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src, obj, defines, save_temps, verbose):
    cmd = [hipcc(), *HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src),
           "-o", obj]
    if save_temps:
        cmd.append("-save-temps=obj")
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=save_temps or None)
    return obj


def build(defines=(), save_temps: str | None = None, out: str = LIB, verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], defines, save_temps, verbose),
                    zip(SOURCES, objs)))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp,
           *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    if out == LIB:
        build_bw(verbose)
    return out


def build_bw(verbose: bool = False) -> str:
    """The bandwidth-reference read kernel bench.py times (a library of its own)."""
    tmp = BW_LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-shared", "-o", tmp, os.path.join(CSRC, "bw_read.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, BW_LIB)
    return BW_LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-D", dest="defines", action="append", default=[])
    ap.add_argument("--save-temps", default=None)
    ap.add_argument("--out", default=LIB)
    args = ap.parse_args(argv)
    print(build(args.defines, args.save_temps, args.out, verbose=True))


if __name__ == "__main__":
    sys.exit(main())
