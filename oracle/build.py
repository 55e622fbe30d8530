"""Build the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure only: the product library never links or loads it.
Flags: -ffp-contract=off and no fast-math, so every fp32 operation in the oracle is
one IEEE operation in the order written; OpenMP splits only the block loop.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bitopt_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fno-strict-aliasing",
          "-fopenmp", "-fPIC", "-shared", "-fvisibility=hidden", "-Wall", "-Wextra"]


def build(force: bool = True, extra_flags=(), out: str = LIB, src: str = SRC) -> str:
    """Compile the oracle (or another source, e.g. a mutant in a test); returns the
    path of the shared library."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(force=True, extra_flags=sys.argv[1:]))
