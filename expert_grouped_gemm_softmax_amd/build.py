"""Build libmoe_mi355x.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# measured-ceiling microkernels for the benchmark, kept out of the layer's library
CALIB_SRC = os.path.join(PKG, "calib", "calibrate.hip")
CALIB_PATH = os.path.join(PKG, "libmoe_calib.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 instructions in any generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _hipcc(srcs: list[str], out: str, verbose: bool) -> None:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if errs and verbose:
        print("\n".join(errs))
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _hipcc(sources(), LIB_PATH, verbose)
    _hipcc([CALIB_SRC], CALIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
