"""Compile the HIP library ``librmsnorm_mi355x.so`` for gfx950 with hipcc.

Runs on a machine without a GPU (hipcc cross-compiles). The result is written
next to this file, where the Python binding loads it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librmsnorm_mi355x.so")
SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "capi.cpp")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(out=LIB, extra_flags=()):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra_flags, *SOURCES, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
