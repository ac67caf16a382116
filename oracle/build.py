"""Build the CPU oracle (plain C, gcc) into oracle/libref_gemm.so.

Test infrastructure only. `-ffp-contract=off` keeps every multiply and add a
separate IEEE operation; no fast-math, so the k-ascending sum is not
reassociated.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ref_gemm.c")
LIB = os.path.join(HERE, "libref_gemm.so")


def build(verbose: bool = False) -> str:
    # A temporary name per process: concurrent builds (parallel test workers)
    # each rename a complete library into place.
    tmp = f"{LIB}.tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
