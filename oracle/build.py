"""Builds the CPU oracle library ``oracle/libnf4ref.so`` with gcc.

Test infrastructure: the oracle is the plain CPU reference the GPU library is
checked against. Flags keep every float operation a single IEEE binary32
operation (no contraction into FMA, no fast-math, SSE arithmetic).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nf4ref.c")
LIB = os.path.join(HERE, "libnf4ref.so")

CFLAGS = [
    "-std=c11",
    "-O2",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-mfpmath=sse",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wextra",
    "-Werror",
]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
