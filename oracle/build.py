"""Builds the CPU oracle shared library (oracle/libsp_oracle.so) with gcc.

TEST INFRASTRUCTURE ONLY.  -ffp-contract=off keeps every fp32 operation of
the elementwise part a separately rounded IEEE operation; no -ffast-math.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sp_oracle.c")
LIB = os.path.join(HERE, "libsp_oracle.so")

CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Werror"]


def build_oracle(out=LIB, extra_flags=()):
    """Compile sp_oracle.c into `out`; returns the path."""
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", out, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build_oracle(*(sys.argv[1:2] or [LIB])))
