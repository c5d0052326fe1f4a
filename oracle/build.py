"""Build the CPU oracle (plain C, fp64, OpenMP) into oracle/libkvd_oracle.so.

Test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline leg load the result.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libkvd_oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "kvd_oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
