"""Build the CPU oracle shared library (plain C, gcc, OpenMP, no fast-math).

Test infrastructure: compiled by ``__graft_entry__.build()`` so the checker
exists wherever the tests run; nothing on the product path loads it.
"""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "mla_oracle.c")


def library_path() -> str:
    return os.path.join(_HERE, "libmla_oracle.so")


def build() -> str:
    out = library_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-fno-fast-math", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
