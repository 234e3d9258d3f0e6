"""Build the HIP library (libqsmoe.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqsmoe.so")
SOURCES = ["qs_moe.hip"]
HEADERS = ["qs_big.h", "qs_kernels.h", "qs_layout.h", "qs_persist.h", "qs_wave.h"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    # The persistent kernel is one long loop over layers whose body is every
    # step of the path; hoisting loop-invariant machine code out of it keeps
    # per-phase values live across all phases and spills to scratch.
    "-mllvm", "-disable-machine-licm",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


# The profiling variant: the same sources with phase stamps compiled in
# (thread 0 of each workgroup records the wall clock at phase boundaries;
# read back by phase_stamps.py).  Never loaded unless asked for.
LIB_STAMPS = os.path.join(PKG, "libqsmoe_stamps.so")


def build_library(verbose: bool = False, stamps: bool = False) -> str:
    """Compile every source into libqsmoe.so (stamps: libqsmoe_stamps.so);
    returns its path."""
    out = LIB_STAMPS if stamps else LIB
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(["-DQS_STAMPS"] if stamps else []), "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError("hipcc failed building libqsmoe.so")
    warn = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if warn and verbose:
        sys.stderr.write(warn + "\n")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True, stamps="--stamps" in sys.argv[1:]))
