"""AddressSanitizer and UndefinedBehaviorSanitizer on the CPU side: the oracle
and the host code of the HIP library (argument checks, dispatch rules, launch
set-up) are rebuilt with both sanitizers, and the CPU tests that exercise
them -- the C-ABI checks, the kernel selection report over the whole shape
grid and every oracle pin (in its quick form) -- run against those builds in a
child process with the clang sanitizer runtime preloaded.  No GPU is used:
every C-ABI call in those tests is rejected before any HIP call, and the
selection report makes none.  A planted heap overflow in a throwaway library
checks first that the runtime reports errors at all."""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.fixture(scope="module")
def san_env(tmp_path_factory):
    rt = _runtime()
    if rt is None or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no ROCm clang sanitizer runtime in this image")
    d = tmp_path_factory.mktemp("san")
    sys.path.insert(0, ROOT)
    from oracle import build as obuild
    from w4a16_dequant_gemv_amd import build as hbuild
    orc = obuild.build_sanitized(str(d / "liboracle_san.so"))
    lib = hbuild.build_host_sanitized(str(d / "libw4a16_san.so"), str(d / "obj"))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", W4A16_LIB=lib, ORACLE_LIB=orc,
               PINS_QUICK="1")
    return d, env


def test_runtime_reports_a_planted_overflow(san_env):
    d, env = san_env
    src = d / "planted.c"
    src.write_text(textwrap.dedent("""
        #include <stdlib.h>
        int planted_read_past_end(int n) { int *a = malloc(n * sizeof(int)); int v = a[n]; free(a); return v; }
    """))
    so = d / "libplanted.so"
    subprocess.run(["/opt/rocm/llvm/bin/clang", "-shared", "-fPIC", "-g", "-fsanitize=address", "-o", str(so),
                    str(src)], check=True)
    code = f"import ctypes; ctypes.CDLL({str(so)!r}).planted_read_past_end(7)"
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 23 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


def test_cpu_suite_under_sanitizers(san_env):
    d, env = san_env
    check = ("import oracle, os; from w4a16_dequant_gemv_amd import _lib; _lib.lib(); o = oracle.load(); "
             "maps = open('/proc/self/maps').read(); "
             "assert _lib.LIB_PATH in maps and o.path in maps and 'libclang_rt.asan' in maps")
    subprocess.run([sys.executable, "-c", check], env=env, cwd=ROOT, check=True, timeout=120)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        "tests/test_abi_cpu.py", "tests/test_dispatch_coverage.py", "tests/test_oracle_pins.py"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
