"""Build the CPU oracle (plain C, fp64) into ``oracle/liboracle.so``.

TEST INFRASTRUCTURE: the oracle is the checker, not the product. Building it
is part of ``__graft_entry__.build()``; only the tests, the smoke check and the
benchmark's CPU-baseline leg load it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# Strict IEEE arithmetic: no fast-math, no contraction of a*b+c into an FMA, so
# every fp64 operation in oracle.c rounds exactly as written.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Werror"]


def build(out=LIB, extra_flags=(), src=SRC):
    """Compile ``src`` with gcc into the shared library ``out``."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
