"""Build the CPU oracle (test infrastructure only) with the host C compiler.

The oracle is plain C99 compiled by gcc with floating-point contraction off,
so every binary32 product and sum in the combine reference is rounded on its
own. It links nothing from the GPU library and includes no HIP header.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ep_oracle.c")
LIB = os.path.join(HERE, "liboracle_ep.so")

CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared"]


def build(cc: str = "gcc", out: str = LIB) -> str:
    """Compile ep_oracle.c into a shared library and return its path."""
    tmp = out + ".tmp"
    subprocess.run([cc, *CFLAGS, "-o", tmp, SRC], check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
