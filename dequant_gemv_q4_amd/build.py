"""Build libqgemv.so (HIP for gfx950) in-tree with hipcc.

    python -m dequant_gemv_q4_amd.build            # build (always recompiles)
    python -m dequant_gemv_q4_amd.build --save-temps DIR   # also keep the gfx950 assembly

Extra preprocessor definitions for tuning sweeps can be passed with ``-D NAME=VALUE``.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqgemv.so")
SOURCES = [os.path.join(CSRC, "gemv_kernels.hip"), os.path.join(CSRC, "abi.cpp")]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
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


def build(defines=(), save_temps: str | None = None, out: str = LIB, verbose: bool = False) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS]
    for d in defines:
        cmd += ["-D", d]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd += ["-save-temps=obj"]
    tmp = out + ".tmp"
    cmd += ["-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    cwd = save_temps if save_temps else None
    subprocess.run(cmd, check=True, cwd=cwd)
    os.replace(tmp, out)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-D", dest="defines", action="append", default=[])
    ap.add_argument("--save-temps", default=None)
    ap.add_argument("--out", default=LIB)
    args = ap.parse_args(argv)
    print(build(args.defines, args.save_temps, args.out, verbose=True))


if __name__ == "__main__":
    sys.exit(main())
