"""Build the CPU oracle (plain C, fp64, OpenMP) into oracle/libkvd_oracle.so.

Test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline leg load the result.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libkvd_oracle.so")


# AddressSanitizer and UndefinedBehaviorSanitizer, every finding fatal
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False, out: str = None) -> str:
    """Compile kvd_oracle.c into `out` (default oracle/libkvd_oracle.so);
    with `sanitize`, instrumented for ASan and UBSan (load it with gcc's
    libasan preloaded)."""
    src = os.path.join(HERE, "kvd_oracle.c")
    lib = out or LIB
    tmp = lib + ".tmp"
    cmd = ["gcc", "-std=c11", "-O1" if sanitize else "-O2", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra"] + (SANITIZE if sanitize else []) + ["-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
