"""Build the CPU oracle (test infrastructure) into oracle/_build/liboracle.so.

The oracle is plain C compiled with gcc: no fused multiply-add contraction
and no fast-math, so that the fp32 statistic operations it names are single
IEEE round-to-nearest-even operations.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lynx_oracle.c")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "liboracle.so")

CFLAGS = [
    "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
    "-Wall", "-Wextra", "-shared", "-fPIC",
]


def build(force: bool = True) -> str:
    """Compile the oracle; returns the path of the shared library."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
