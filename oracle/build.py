"""Build the CPU oracle library (oracle/liboracle.so) with gcc.

Test infrastructure: the oracle is a checker, built next to the product so the
tests can load it; nothing in the product path links it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = [os.path.join(HERE, "oracle.c")]
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add, every operation rounds once in
# source order.  No -ffast-math: libm cos/sin and IEEE semantics are kept.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, "-o", tmp, *SOURCES, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
