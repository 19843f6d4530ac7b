"""Builds the CPU oracle (test infrastructure) with gcc: liboracle.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]


def build() -> str:
    src = os.path.join(HERE, "oracle.c")
    tmp = LIB + ".tmp"
    subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, src, "-lm"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
