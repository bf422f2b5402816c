"""Compile the HIP sources of this package into libmla_amd.so (gfx950 only).

    python -m mla_latent_cache_amd.build

Each translation unit is compiled by hipcc into an object under _build/ and the
objects are linked into mla_latent_cache_amd/libmla_amd.so.  Packed-FP32 VALU
instructions are disabled for every device compilation.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["decode.hip", "decode_flat.hip", "gemm.hip", "prolog.hip", "prefill.hip", "prefill_attend.hip", "mlaprolog.hip",
           "mla_api.cpp"]
LIB = os.path.join(PKG, "libmla_amd.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Per-source additions.  The prefill attention kernel keeps 128 accumulator
# registers across its tile loop and rescales them (vector work) on a rare
# branch; with the matrix-register form of the MFMA the compiler copies all of
# them to vector registers on every tile.  The vector-register form keeps them
# where the vector unit can reach them, with bitwise-identical results.  The
# prefill decompression GEMM (64 accumulator registers per lane) was tuned with
# the same form.
EXTRA_FLAGS = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "prefill_attend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + FLAGS + EXTRA_FLAGS.get(src, [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
