"""Build the float64 CPU oracle (test infrastructure) into oracle/libvlf_oracle.so with gcc.

Plain -O2, OpenMP, no fast-math and no floating-point contraction, so every operation rounds
as written.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "vlf_oracle.c")
LIBRARY = os.path.join(HERE, "libvlf_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
        "-fno-fast-math", "-Wall", "-Wextra", SOURCE, "-o", LIBRARY + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIBRARY + ".tmp", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
