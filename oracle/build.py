"""Builds the test-only oracle library (oracle/liboracle.so) with gcc.

The oracle is test infrastructure: only tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg load it.  It is plain host C with no HIP header.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_gemm.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile `src` into the shared library `out` and return its path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra_flags, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
