"""Build the CPU oracle (test infrastructure only): gcc, fp64, OpenMP.

Run as ``python -m oracle.build`` or call ``build()``.  The shared object is
written next to this file and is git-ignored.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tq_oracle.c")
LIB = os.path.join(HERE, "libtq_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-fvisibility=hidden", "-ffp-contract=off", "-D_GNU_SOURCE",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
