"""Builds libtgemm.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

The library is built in-tree, next to this file, so that the built code
travels with the source tree.  Every HIP compile line carries
`-Xclang -target-feature -Xclang -packed-fp32-ops`, which keeps the compiler
from emitting packed-fp32 VALU instructions.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtgemm.so")
# measurement program: MFMA issue rate and clock on every SIMD (bench.py --mfma-ceiling)
CEILING_SRC = os.path.join(CSRC, "mfma_ceiling.hip")
CEILING_BIN = os.path.join(HERE, "mfma_ceiling")
SOURCES = [os.path.join(CSRC, "tgemm.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def build(out: str = LIB, extra=(), verbose: bool = False) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *HIPFLAGS, *extra, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32-ops feature and says so
    noise = "packed-fp32-ops"
    msg = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
    if msg.strip() and verbose:
        print(msg, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build_ceiling(out: str = CEILING_BIN, verbose: bool = False) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", CEILING_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_ceiling(verbose=True))
