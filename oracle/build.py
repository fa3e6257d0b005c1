"""Build the CPU oracle library ``oracle/libcsa2ref.so`` with the host C compiler.

Test infrastructure only: the oracle is compiled here so that the tests, the
smoke check and the benchmark's CPU-baseline leg can load it.  Plain gcc, no
HIP headers, no code shared with the device library.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libcsa2ref.so")
SRC = os.path.join(HERE, "csa2_ref.c")


def build(verbose: bool = False) -> str:
    cmd = [
        os.environ.get("CC", "gcc"), "-std=c11", "-O3", "-fopenmp", "-fPIC", "-shared",
        "-Wall", "-Wextra", "-Wno-unused-parameter",
        SRC, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
