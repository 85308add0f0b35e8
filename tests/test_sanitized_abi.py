"""The C-ABI tests (tests/test_abi.py) again, against a build of the library
whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer
(libflashsk_san.so: `python streaming_sinkhorn_solver_log_amd/build.py
--sanitize`, also made by __graft_entry__.build()). Every validation path runs
with the sanitizer runtime preloaded; any report aborts the run. No GPU is
used: every call fails validation before its first HIP call."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "streaming_sinkhorn_solver_log_amd", "libflashsk_san.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _asan_runtime():
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_abi_validation_under_address_and_undefined_behavior_sanitizers():
    if not os.path.exists(SAN_LIB):
        pytest.skip("libflashsk_san.so is not built (build.py --sanitize)")
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("no shared AddressSanitizer runtime next to hipcc")
    env = dict(os.environ, LD_PRELOAD=runtime, FLASHSK_ABI_LIB=SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert " passed" in r.stdout
