"""Compile the CPU oracle (plain C, gcc) into oracle/liboracle.so.

TEST INFRASTRUCTURE ONLY: the oracle is the checker for the HIP library, and
building it is part of building the checker, never part of the library.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add, so every product and sum rounds in
# fp64 exactly as written; no -ffast-math, so IEEE semantics hold.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
          "-Wall", "-Wextra"]


def build(src=SRC, out=LIB, extra=()):
    """Compile `src` to the shared library `out`; returns `out`."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(), file=sys.stderr)
