"""Build the CPU oracle (oracle/oracle.c -> oracle/liboracle.so) with gcc.

Test infrastructure only: the product library never links or loads it.
-ffp-contract=off keeps every FP32 product and sum separately rounded, as the
oracle's arithmetic is written; no -ffast-math.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra"]


def build(src=SRC, out=LIB, extra=()):
    """Compile src into the shared library out; returns out."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
