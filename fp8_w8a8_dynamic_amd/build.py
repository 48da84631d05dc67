"""Build the HIP library ``libfp8w8a8.so`` in-tree for gfx950.

Usage: ``python -m fp8_w8a8_dynamic_amd.build`` (or ``build()`` from Python).
Every call compiles all sources again: hipcc cross-compiles gfx950 code
without a GPU.  Objects go to ``_build/`` at the repository root; the shared
library lands next to this file, where the binding loads it.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libfp8w8a8.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["api.cpp", "quant.hip", "norm.hip", "swiglu.hip", "kvcache.hip",
           "gemm.hip", "gemv.hip", "tokgroup.hip"]

# The benchmark's measured-peak kernels, a library of their own.
PEAKS_SOURCES = ["peaks.hip"]
PEAKS_LIB_PATH = os.path.join(PKG_DIR, "libfp8w8a8_peaks.so")

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
# No fast-math and no denormal flushing: the quantizer must see IEEE float32
# division and subnormal scales exactly as the format definition says.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-I", os.path.join(ROOT, "include"),
]


# Host-side sanitizer build (CPU tests of the argument validation): every
# -fsanitize= applies to host code only (-Xarch_host); device code is built
# as usual and never runs in those tests.
SANITIZE_FLAGS = [f for opt in ("-fsanitize=address", "-fsanitize=undefined",
                                "-fno-sanitize-recover=all",
                                "-fno-omit-frame-pointer")
                  for f in ("-Xarch_host", opt)]
SANITIZED_DIR = os.path.join(BUILD_DIR, "sanitized")
SANITIZED_LIB_PATH = os.path.join(SANITIZED_DIR, "libfp8w8a8_asan_ubsan.so")


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required")
    return path


def _compile(src: str, out_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n"
                           f"{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, path, extra=()):
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs,
           "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every source, link the library and the benchmark's peaks
    library; return the library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PEAKS_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB_PATH)
    _link([objs[s] for s in PEAKS_SOURCES], PEAKS_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
        print(f"built {PEAKS_LIB_PATH}")
    return LIB_PATH


def build_sanitized(verbose: bool = False) -> str:
    """The library with AddressSanitizer and UndefinedBehaviorSanitizer on its
    host code (for CPU tests of the C ABI's validation; loaded with the
    sanitizer runtime preloaded, see sanitizer_runtime()).  Returns its path."""
    os.makedirs(SANITIZED_DIR, exist_ok=True)
    extra = ["-g", *SANITIZE_FLAGS]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, SANITIZED_DIR, extra), SOURCES))
    _link(objs, SANITIZED_LIB_PATH, SANITIZE_FLAGS)
    if verbose:
        print(f"built {SANITIZED_LIB_PATH}")
    return SANITIZED_LIB_PATH


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (which carries
    the UndefinedBehaviorSanitizer handlers), to preload into a process
    that loads the sanitized library."""
    res = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the compiler's libclang_rt.asan-x86_64.so was not found")
    return path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
