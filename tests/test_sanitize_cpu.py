"""CPU sanitizer job: the host side of libbdattn (planner, work orders,
argument validation, workspace carving) and the oracle, built with
AddressSanitizer and UndefinedBehaviorSanitizer (the device code is
unchanged), run the host tests (ABI contract, work-order balance, oracle
pins) in a child process with the sanitizer runtime preloaded.

Two checks keep the job honest: a canary object with a heap overflow must
abort under the same flags and runtime, and the child asserts that the
sanitized libraries are the ones mapped into it."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HOST_TESTS = ["tests/test_abi_cpu.py", "tests/test_plan_balance.py", "tests/test_oracle_pins.py",
              "tests/test_rowstats_oracle.py"]


def _runtime():
    rts = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                        "libclang_rt.asan-x86_64.so")))
    if not rts:
        pytest.skip("clang sanitizer runtime not found")
    return rts[-1]


def _env(d, rt):
    return dict(os.environ, BDATTN_SANITIZED_DIR=str(d), LD_PRELOAD=rt,
                ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


CANARY = r"""
#include <stdlib.h>
int canary(int i) { int* p = (int*)malloc(4 * sizeof(int)); int v = p[i]; free(p); return v; }
"""


def test_sanitizer_canary_fires(tmp_path):
    rt = _runtime()
    src = tmp_path / "canary.c"
    src.write_text(CANARY)
    so = tmp_path / "libcanary.so"
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    subprocess.run([clang, "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined", "-shared-libsan",
                    "-o", str(so), str(src)], check=True)
    code = f"import ctypes; print(ctypes.CDLL({str(so)!r}).canary(7))"
    r = subprocess.run([sys.executable, "-c", code], env=_env(tmp_path, rt), capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_host_code_under_sanitizers(tmp_path):
    rt = _runtime()
    from block_diffusion_lm_bdlm_amd import build as lb
    from oracle import build as ob
    lb.build_sanitized(str(tmp_path))
    ob.build_sanitized(str(tmp_path))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-v", "-m", "not gpu", "-p", "no:cacheprovider"]
                       + HOST_TESTS, cwd=ROOT, env=_env(tmp_path, rt), capture_output=True, text=True,
                       timeout=900)
    tail = (r.stdout[-3000:] + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "test_sanitized_libraries_loaded PASSED" in r.stdout, tail
