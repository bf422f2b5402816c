"""The C-ABI host validation paths under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; no GPU is touched).

mla_api.cpp -- every argument check of the boundary -- is compiled with the
host sanitizers and linked with the ordinary objects of the other sources into
a separate library; tests/test_abi_host.py then runs against it in a child
process that preloads the sanitizer runtime.  Any report (a bad read or write,
an invalid enum or shift, an overflowing signed product) fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(BUILD, "sanitized")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
sys.path.insert(0, ROOT)
from mla_latent_cache_amd import build as _build  # noqa: E402  (the library's own source list)

OTHERS = [s for s in _build.SOURCES if s != "mla_api.cpp"]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _runtime():
    if not os.path.exists(CLANG):
        return None
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_host_validation_is_clean_under_asan_and_ubsan():
    objs = [os.path.join(BUILD, s + ".o") for s in OTHERS]
    rt = _runtime()
    if shutil.which(HIPCC) is None or rt is None or not all(os.path.exists(o) for o in objs):
        pytest.skip("needs hipcc, the sanitizer runtime and the objects of a library build")
    os.makedirs(OUT, exist_ok=True)
    api_o = os.path.join(OUT, "mla_api.o")
    lib = os.path.join(OUT, "libmla_amd_sanitized.so")
    csrc = os.path.join(ROOT, "mla_latent_cache_amd", "csrc")
    subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++20", "-fPIC",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    f"-I{os.path.join(ROOT, 'include')}", f"-I{csrc}", *HOST_SAN,
                    "-c", os.path.join(csrc, "mla_api.cpp"), "-o", api_o], check=True, capture_output=True)
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *HOST_SAN[:4], "-shared-libsan",
                    "-o", lib, api_o, *objs], check=True, capture_output=True)
    env = dict(os.environ, MLA_AMD_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"),
                        "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
