"""The C ABI's host code under AddressSanitizer.

api.cpp is rebuilt with the sanitizer on its host code only (the kernel
objects are the release ones), loaded into a Python process that preloads the
sanitizer runtime, and the whole host-side ABI suite (test_abi_cpu.py: every
exported symbol, host validation of every field, null-handle paths, the
no-GPU error path) runs against it.  Any invalid access in the host code
aborts that process with the sanitizer's report."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _env(lib, rt):
    env = dict(os.environ)
    env["MLA_DECODE_LIB_PATH"] = lib
    env["LD_PRELOAD"] = rt
    # the interpreter's own allocations are outside the library under test
    env["ASAN_OPTIONS"] = "detect_leaks=0:exitcode=86"
    return env


def test_abi_host_code_under_address_sanitizer():
    if not shutil.which("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc is not installed")
    from mla_latent_cache_decode_amd.build import asan_runtime, build_asan_host
    rt = asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime")
    lib = build_asan_host()
    env = _env(lib, rt)
    # the binding loads the sanitized build
    probe = subprocess.run([sys.executable, "-c", "import mla_latent_cache_decode_amd as m; "
                            "print(m.load_library()._name)"], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=600)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.strip().endswith("libmla_decode_asan.so"), probe.stdout
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                          "tests/test_abi_cpu.py"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
