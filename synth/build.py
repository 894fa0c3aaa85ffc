"""Compile the seeded input generator into synth/libsynth.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "synth.c")
    out = os.path.join(HERE, "libsynth.so")
    cmd = ["gcc", "-O2", "-std=gnu11", "-fopenmp", "-shared", "-fPIC", "-Wall", src, "-o", out, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    build(verbose=True)
