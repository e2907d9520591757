"""Compile the CPU oracle (plain C, IEEE double, OpenMP) into oracle/libhs_oracle.so.

Test infrastructure only: the product library never links or loads this.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "libhs_oracle.so")


def build(verbose=False):
    src = os.path.join(HERE, "hs_oracle.c")
    tmp = SO + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
