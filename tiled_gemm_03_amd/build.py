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
# the host code and the kernel units (compiled in parallel, then linked)
SOURCES = [os.path.join(CSRC, f) for f in (
    "tgemm.hip", "k_tiled_big.hip", "k_tiled_mid.hip", "k_tiled_small.hip", "k_tiled_tiny.hip", "k_tiled_f32.hip",
    "k_ring_big.hip", "k_ring_mid.hip", "k_ring_small.hip", "k_ring_small_fused.hip", "k_direct.hip",
    "k_tiled_big_fused.hip", "k_ring_big_fused.hip", "k_ring_mid_fused.hip", "k_direct_fused.hip",
    "k_ring_big_kt.hip", "k_ring_mid_kt.hip", "k_ring_big_fused_kt.hip", "k_ring_mid_fused_kt.hip",
    "k_ring_big_fp8.hip", "k_ring_big_fp8_kt.hip", "k_ring_mid_fp8.hip", "k_ring_small_fp8.hip", "k_direct_fp8.hip",
    "k_splitk.hip", "attention.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32-ops feature and says so
    msg = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln)
    return r.returncode, msg


def build(out: str = LIB, extra=(), verbose: bool = False, jobs: int = 0) -> str:
    """Compiles every source to an object (in parallel), then links them."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = jobs or max(1, min(len(SOURCES), os.cpu_count() or 1))
    tag = "%d" % os.getpid()
    objs = [os.path.join(HERE, "_obj_" + os.path.splitext(os.path.basename(src))[0] + "." + tag + ".o")
            for src in SOURCES]
    compile_flags = [f for f in HIPFLAGS if f != "-shared"] + ["-c"]
    cmds = [[HIPCC, *compile_flags, *extra, src, "-o", obj] for src, obj in zip(SOURCES, objs)]
    try:
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_hipcc, cmds))
        for cmd, (rc, msg) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd), flush=True)
            if rc != 0:
                raise RuntimeError(f"hipcc failed ({rc}) on {cmd[-3]}:\n{msg}")
            if msg.strip() and verbose:
                print(msg, file=sys.stderr)
        tmp = out + ".tmp" + tag
        link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        rc, msg = _hipcc(link)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{msg}")
        os.replace(tmp, out)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
