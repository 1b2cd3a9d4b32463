"""Build the fp64 CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

Flags: -O2 with OpenMP; -ffp-contract=off and no -ffast-math so that every product and sum is
rounded in double precision exactly as written in attention.c.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attention.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(src=SRC, out=LIB, extra_flags=()):
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)
