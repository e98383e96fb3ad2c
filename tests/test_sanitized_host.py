"""The host code of the library and the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

The library's host side (argument checks, workspace sizing, kernel planning,
the status strings) and the C oracle are rebuilt with clang's ASan and UBSan
(UB is fatal), and the CPU suites that exercise them -- the C-ABI host
checks, the oracle's pins, the input generator and the benchmark's
bookkeeping -- run again in a child process with the ASan runtime preloaded.
No kernel is launched.  The builds are cached under _build/sanitized/ by a
hash of their sources and flags.  A first test checks the harness itself:
a throwaway C file that reads past a heap block must abort under it."""
import hashlib
import os
import subprocess
import sys

import pytest

import oracle
from transformer_scaled_dot_attn_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_abi_host.py", "tests/test_oracle_pins.py", "tests/test_workloads.py",
          "tests/test_bench_host.py"]


def _env(libattn=None, liboracle=None):
    env = dict(os.environ)
    env["LD_PRELOAD"] = hip_build.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    if libattn:
        env["TSDA_TEST_LIBATTN"] = libattn
    if liboracle:
        env["TSDA_TEST_LIBORACLE"] = liboracle
    return env


def _digest():
    h = hashlib.sha256()
    h.update(" ".join(hip_build.compile_flags()).encode())
    for d in (hip_build.CSRC, os.path.join(ROOT, "include"), os.path.join(ROOT, "oracle")):
        for f in sorted(os.listdir(d)):
            if f.endswith((".hip", ".cpp", ".h", ".c")):
                h.update(f.encode())
                h.update(open(os.path.join(d, f), "rb").read())
    h.update(open(hip_build.__file__, "rb").read())
    return h.hexdigest()[:16]


@pytest.fixture(scope="module")
def sanitized_builds():
    out = os.path.join(ROOT, "_build", "sanitized", _digest())
    lib = os.path.join(out, "libattn_sanitized.so")
    orc = os.path.join(out, "liboracle_sanitized.so")
    if not (os.path.exists(lib) and os.path.exists(orc)):
        hip_build.build_sanitized(out)
        oracle.compile_oracle_sanitized(orc)
    return lib, orc


def test_sanitizer_harness_catches_a_heap_overflow(tmp_path):
    src = tmp_path / "overflow.c"
    src.write_text("#include <stdlib.h>\n"
                   "int read_past(int n) { int* a = malloc(sizeof(int) * n); int v = a[n];\n"
                   "  free(a); return v; }\n")
    lib = tmp_path / "liboverflow.so"
    subprocess.run(["/opt/rocm/llvm/bin/clang", "-O0", "-g", "-fPIC", "-shared",
                    "-fsanitize=address", str(src), "-o", str(lib)], check=True)
    code = f"import ctypes; ctypes.CDLL({str(lib)!r}).read_past(4)"
    res = subprocess.run([sys.executable, "-c", code], env=_env(), capture_output=True,
                         text=True)
    assert res.returncode != 0 and "heap-buffer-overflow" in res.stderr, res.stderr[-2000:]


def test_host_suites_under_sanitizers(sanitized_builds):
    lib, orc = sanitized_builds
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "-p", "no:xdist", "-m", "not gpu"] + SUITES,
                         cwd=ROOT, env=_env(lib, orc), capture_output=True, text=True,
                         timeout=1200)
    tail = (res.stdout[-3000:] + res.stderr[-3000:])
    assert res.returncode == 0, tail
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, tail
    assert " passed" in res.stdout and "failed" not in res.stdout, tail
