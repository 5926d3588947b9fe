"""Compile the HIP library ``librmsnorm_mi355x.so`` for gfx950 with hipcc;
``libstream_floor.so``, the benchmark's streaming-floor kernel (the
backward's row traffic through the same window ring, without its arithmetic;
not part of the C ABI); and ``_autograd_ext``, the torch C++ autograd nodes
of the autograd wrappers, with the host compiler against torch's headers
(HIP host API only, no device code), linked to the library.

Runs on a machine without a GPU (hipcc cross-compiles). The results are
written next to this file, where the Python binding and the benchmark load
them.
"""
import os
import subprocess
import sysconfig

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librmsnorm_mi355x.so")
SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "long_rows.hip"), os.path.join(CSRC, "capi.cpp")]
FLOOR_LIB = os.path.join(HERE, "libstream_floor.so")
FLOOR_SOURCES = [os.path.join(CSRC, "stream_floor.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(sources, out, extra_flags):
    tmp = out + ".tmp"
    subprocess.run([HIPCC, *FLAGS, *extra_flags, *sources, "-o", tmp], check=True)
    os.replace(tmp, out)
    return out


EXT_SOURCE = os.path.join(CSRC, "autograd_ext.cpp")
EXT = os.path.join(HERE, "_autograd_ext" + sysconfig.get_config_var("EXT_SUFFIX"))


def build_ext(out=EXT):
    """The autograd nodes: a Python extension module built with the host C++
    compiler against torch's headers and libraries, linked to the library
    next to it (found through an $ORIGIN run path)."""
    import torch
    import torch.utils.cpp_extension as ce
    cxx = os.environ.get("CXX", "g++")
    abi = int(torch._C._GLIBCXX_USE_CXX11_ABI)
    cmd = [cxx, "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wno-unused-function",
           "-D__HIP_PLATFORM_AMD__=1", "-DUSE_ROCM=1", f"-D_GLIBCXX_USE_CXX11_ABI={abi}",
           "-DTORCH_EXTENSION_NAME=_autograd_ext", "-DTORCH_API_INCLUDE_EXTENSION_H",
           *[f"-I{p}" for p in ce.include_paths()], "-I", sysconfig.get_paths()["include"],
           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           EXT_SOURCE, "-o", out + ".tmp",
           "-L", HERE, "-lrmsnorm_mi355x", "-Wl,-rpath,$ORIGIN",
           *[f"-L{p}" for p in ce.library_paths()], "-lc10", "-lc10_hip", "-ltorch", "-ltorch_cpu",
           "-ltorch_python", "-L/opt/rocm/lib", "-lamdhip64"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build(out=LIB, extra_flags=(), floor=True, ext=True):
    """Build the library (and, unless turned off, the floor kernel's library
    and the autograd extension)."""
    _compile(SOURCES, out, extra_flags)
    if floor:
        _compile(FLOOR_SOURCES, FLOOR_LIB, extra_flags)
    if ext and out == LIB:
        build_ext()
    return out


if __name__ == "__main__":
    print(build())
