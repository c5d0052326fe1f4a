"""Build libkvd.so (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m kv_cached_decode_amd.build        # or build() from Python

Every HIP source is compiled with packed fp32 instructions disabled
(-target-feature -packed-fp32-ops) and linked into one shared library next to
this file, where the Python binding loads it.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvd.so")
BUILD_DIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["kvd.cpp", "rope_append.hip", "attn_valu.hip", "attn_mfma.hip", "attn_prefill.hip",
           "attn_combine.hip", "stream_probe.hip", "check_descriptor.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


# Host code only (the device code is never instrumented): AddressSanitizer
# and UndefinedBehaviorSanitizer with the shared ASan runtime, which a
# process preloads to load the library.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-shared-libasan", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _compile(src, verbose, build_dir, extra):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC] + lang + COMMON + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize_host: bool = False, out: str = None) -> str:
    """Compile libkvd.so into `out` (default next to this file); with
    `sanitize_host`, the host code is instrumented (a separate build folder)."""
    lib = out or LIB
    extra = SANITIZE_HOST if sanitize_host else []
    build_dir = BUILD_DIR + ("_sanitize" if sanitize_host else "")
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + extra + ["-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
