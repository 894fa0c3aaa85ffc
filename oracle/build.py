"""Compile the oracle (plain C, OpenMP) into oracle/liboracle.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "oracle.c")
    out = os.path.join(HERE, "liboracle.so")
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra", src, "-o", out, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    build(verbose=True)
