"""Builds libflashsk.so in-tree from csrc/*.hip with hipcc for gfx950, and the
unit-rate microbenchmarks peaks/libskpeaks.so that `bench.py --peaks` runs.

Usage: python streaming_sinkhorn_solver_log_amd/build.py   (or build_library()).
Run it as a script: importing the package needs the library it builds.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libflashsk.so")
OBJ_DIR = os.path.join(PKG, "_build")
PEAKS_SRC = os.path.join(PKG, "peaks", "peaks.hip")
PEAKS_LIB = os.path.join(PKG, "peaks", "libskpeaks.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed FP32 instructions stay disabled: this code base relies on plain
# float arithmetic and does not emit them.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the C-ABI
# validation layer (device code is built as usual: each -fsanitize= applies to
# the host pass only). The result, libflashsk_san.so, is loaded by
# tests/test_sanitized_abi.py with the sanitizer runtime preloaded.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
SAN_LIB = os.path.join(PKG, "libflashsk_san.so")
SAN_OBJ_DIR = os.path.join(PKG, "_build_san")


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_OBJ_DIR if sanitize else OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *(SAN_FLAGS if sanitize else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build_library(jobs: int = 8, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    os.makedirs(SAN_OBJ_DIR if sanitize else OBJ_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), srcs))
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *(SAN_FLAGS if sanitize else []),
           "-Xarch_host", "-shared-libsan", "-o", tmp, *objs] if sanitize else \
          [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)
    return out


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (preloaded by the sanitized tests)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build_peaks() -> str:
    """Compiles the microbenchmark library (separate from libflashsk.so)."""
    tmp = PEAKS_LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, "-shared", PEAKS_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PEAKS_SRC}:\n{err}")
    os.replace(tmp, PEAKS_LIB)
    return PEAKS_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        print(build_library(sanitize=True))
    else:
        print(build_library())
        print(build_peaks())
