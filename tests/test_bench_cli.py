"""Host-side checks of the command line and the loader (no GPU needed): bench.py
refuses a request for more than one GPU with a message and a non-zero status
before anything touches a device, and a missing library makes the first entry
point raise (there is no other way to compute)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_help_lists_the_contract_flags():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout


def test_missing_library_fails_loudly():
    # A fresh interpreter with the library path pointed at nothing: the first
    # entry point raises instead of computing anything another way.
    code = ("import mla_latent_cache_amd._binding as b\n"
            "b.LIB_PATH = '/nonexistent/libmla_amd.so'\n"
            "try:\n"
            "    b.mla_default_scale((64, 192, 64, 256, 512))\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "is missing" in r.stdout
