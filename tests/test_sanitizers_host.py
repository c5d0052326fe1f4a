"""The oracle and the host side of libkvd.so under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU (no GPU needed).

The oracle pins run against an instrumented build of oracle/kvd_oracle.c
(gcc), and the C-ABI host tests against a build of libkvd.so whose host code
is instrumented (clang, through hipcc; validation, planning and workspace
sizing -- every case fails or answers before a kernel would launch).  Each
runs in a child process that preloads the matching ASan runtime; every
finding is fatal there (UBSan does not recover), so it fails the child and
this test.  Leak checking is off: the Python interpreter and the HIP runtime
keep allocations until exit by design."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _child(env_extra, tests):
    env = dict(os.environ)
    env.update(env_extra)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + tests
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-5000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-5000:]
    return out


def _preload(runtime):
    prev = os.environ.get("LD_PRELOAD", "")
    return runtime + (" " + prev if prev else "")


ASAN_OPTIONS = "detect_leaks=0:alloc_dealloc_mismatch=0:verify_asan_link_order=0:abort_on_error=1"


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    import oracle
    lib = oracle.build(sanitize=True, out=str(tmp_path / "libkvd_oracle_asan.so"))
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.isabs(rt), "gcc's libasan not found"
    out = _child({"LD_PRELOAD": _preload(rt), "ASAN_OPTIONS": ASAN_OPTIONS,
                  "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1", "KVD_ORACLE_LIB": lib},
                 ["tests/test_oracle_pins.py"])
    assert " passed" in out


def test_abi_host_under_asan_and_ubsan(tmp_path):
    from kv_cached_decode_amd import build as kbuild
    if not os.path.exists(kbuild.HIPCC):
        pytest.skip("hipcc not available")
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rts:
        pytest.skip("clang's shared ASan runtime not found")
    lib = kbuild.build(sanitize_host=True, out=str(tmp_path / "libkvd_asan.so"))
    out = _child({"LD_PRELOAD": _preload(rts[0]), "ASAN_OPTIONS": ASAN_OPTIONS,
                  "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1", "KVD_LIB_PATH": lib},
                 ["tests/test_abi_host.py"])
    assert " passed" in out


def test_the_harness_catches_a_planted_overflow(tmp_path):
    """Control: a one-element heap overflow in a throwaway instrumented C
    library, called the way the pins call the oracle, must abort the child
    with an AddressSanitizer report."""
    src = tmp_path / "overflow.c"
    src.write_text("#include <stdlib.h>\n"
                   "int overflow(int n) { int *a = malloc(n * sizeof(int)); a[n] = 1; int r = a[0]; free(a); return r; }\n")
    lib = tmp_path / "liboverflow.so"
    subprocess.run(["gcc", "-shared", "-fPIC", "-g", "-fsanitize=address", "-o", str(lib), str(src)], check=True)
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=_preload(rt), ASAN_OPTIONS=ASAN_OPTIONS)
    code = f"import ctypes; ctypes.CDLL({str(lib)!r}).overflow(4)"
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
