"""Build the CPU oracle (test infrastructure) into oracle/libep_oracle.so.

Plain C11 with the host compiler; -ffp-contract=off keeps every floating-point
expression rounding exactly as written.  Usable as a script or imported.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libep_oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "ep_oracle.c")
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-fPIC", "-shared", "-o", LIB + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
