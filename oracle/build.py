"""Build the CPU oracle shared library with gcc.

Test infrastructure only (see tropical_oracle.c).  Flags: -O2, no fast-math,
no FMA contraction, OpenMP over output rows.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tropical_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-fopenmp", "-Wall", "-Wextra"]


def build(src=SRC, out=LIB, quiet=True):
    """Compile `src` into the shared library `out` (always recompiles)."""
    cmd = ["gcc", *CFLAGS, src, "-o", out + ".tmp", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + res.stderr)
    if not quiet and res.stderr:
        sys.stderr.write(res.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
