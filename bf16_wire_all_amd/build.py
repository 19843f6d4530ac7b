"""Builds libxfer.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build", "xfer")
LIB = os.path.join(HERE, "libxfer.so")

SOURCES = ["api.cpp", "stream_pipeline.cpp", "groups.cpp", "pack_combine.hip", "argmax.hip", "runs_copy.hip",
           "descs_copy.hip", "pages.cpp", "pages_copy.hip"]

# -packed-fp32-ops: never emit packed F32 instructions (the host pass warns
# that it does not know the feature; harmless).  No fast-math and no denormal
# flushing: the sums must be IEEE binary32 with subnormals kept.
# Small per-thread arrays (the loads a thread keeps in flight) must live in
# registers, never in LDS.
HIPFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-disable-promote-alloca-to-lds",
            "-fno-gpu-rdc", "-I", os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *HIPFLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-fno-gpu-rdc", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
