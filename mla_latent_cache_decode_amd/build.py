"""Build libmla_decode.so in-tree with hipcc for gfx950.

Usage: python -m mla_latent_cache_decode_amd.build   (or __graft_entry__.build())
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmla_decode.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["decode_bf16.hip", "decode.hip", "decode_mx.hip", "plan_combine.hip", "scratch.hip", "api.cpp"]
# the matrix-core rate and clock probe: a library of its own, outside the decode path
PROBE_SOURCE = "probe_mfma_clock.hip"
PROBE_LIB_PATH = os.path.join(PKG, "libmla_probe.so")

# per-source extra compiler flags
SOURCE_FLAGS: dict = {}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    # code object v5: loadable by the HIP runtime bundled with PyTorch as well
    "-mcode-object-version=5",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # no packed-FP32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every HIP source for gfx950 and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    flags = COMMON_FLAGS + list(extra_flags or [])
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC] + flags + SOURCE_FLAGS.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    probe_tmp = PROBE_LIB_PATH + ".tmp"
    cmds.append([HIPCC] + flags + ["-shared", "-x", "hip", os.path.join(CSRC, PROBE_SOURCE), "-o", probe_tmp])
    # the translation units compile independently: one hipcc each, in parallel
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "0") or 0) or (os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB_PATH)
    os.replace(probe_tmp, PROBE_LIB_PATH)
    return LIB_PATH


def asan_runtime() -> str | None:
    """The clang AddressSanitizer runtime that hipcc's host compiler links against."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_asan_host(verbose: bool = False) -> str:
    """The same library with its host code (the C ABI in api.cpp) built under
    AddressSanitizer; the kernel objects are the release ones.  Load it into a
    process that preloads asan_runtime().  Returns its path."""
    kernels = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(k) for k in kernels):
        build(verbose)
    out_dir = os.path.join(BUILD_DIR, "asan")
    os.makedirs(out_dir, exist_ok=True)
    obj = os.path.join(out_dir, "api.o")
    # -Xarch_host before each sanitizer flag: host code only, never GPU code
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libasan"]
    flags = [f for f in COMMON_FLAGS if f != "-O3"] + ["-O1", "-g"] + san
    _run([HIPCC] + flags + ["-c", os.path.join(CSRC, "api.cpp"), "-o", obj], verbose)
    lib = os.path.join(out_dir, "libmla_decode_asan.so")
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + san + ["-o", lib, obj] + kernels, verbose)
    return lib


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
