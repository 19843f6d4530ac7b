"""Builds the seeded input generators with gcc: libdatagen.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libdatagen.so")


def build() -> str:
    src = os.path.join(HERE, "datagen.c")
    tmp = LIB + ".tmp"
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-fno-fast-math", "-fPIC", "-shared",
                           "-Wall", "-Wextra", "-Werror", "-o", tmp, src, "-lm"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
