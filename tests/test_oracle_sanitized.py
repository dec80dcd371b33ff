"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

oracle.c is compiled with -fsanitize=address,undefined into a temporary
library, and a child pytest process loads it in place of the normal build
(PA_ORACLE_LIB) with the ASan runtime preloaded. That process runs every pin
against the sanitized oracle, then the mutant suite (each mutant compiled as
usual, its pins run in the same sanitized process). Any out-of-bounds access,
use after free or undefined behaviour in the oracle ends the child with a
sanitizer report, which fails this test.
"""
import os
import subprocess
import sys
from pathlib import Path

import pytest

import oracle

ROOT = Path(__file__).resolve().parent.parent
SAN_FLAGS = ("-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g")


def _runtime(name: str) -> str:
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else ""


def test_pins_and_mutants_under_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if not asan:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    lib = oracle.compile_library(oracle.SOURCE, tmp_path / "liboracle_sanitized.so", extra_flags=SAN_FLAGS)
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:exitcode=23"   # the interpreter itself keeps memory until exit
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=24"
    env["PA_ORACLE_LIB"] = str(lib)
    env["OMP_NUM_THREADS"] = "4"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
           "tests/test_oracle_pins.py", "tests/test_oracle_mutants.py"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]


def test_the_harness_reports_a_planted_overflow(tmp_path):
    """The same flags, preload and loading path catch a heap overflow planted in a
    throwaway C function (not the oracle), and the child sees the library it was given."""
    asan = _runtime("libasan.so")
    if not asan:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\n"
                   "int read_past_end(int n) { int* a = malloc(n * sizeof(int)); for (int i = 0; i < n; ++i) a[i] = i;\n"
                   "  int s = a[n]; free(a); return s; }\n")
    lib = oracle.compile_library(src, tmp_path / "libplanted.so", extra_flags=SAN_FLAGS)
    san = oracle.compile_library(oracle.SOURCE, tmp_path / "liboracle_sanitized.so", extra_flags=SAN_FLAGS)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:exitcode=23", PA_ORACLE_LIB=str(san))
    probe = ("import ctypes, oracle; print('loaded', oracle.get().lib._name, flush=True); "
             f"ctypes.CDLL({str(lib)!r}).read_past_end(8)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert f"loaded {san}" in r.stdout, r.stdout + r.stderr[-2000:]
    assert r.returncode == 23 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
