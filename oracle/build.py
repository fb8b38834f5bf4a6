"""Compile the FP64 reference attention (test infrastructure) with gcc.

The oracle is plain C built by the host compiler; it shares nothing with the
GPU library.  ``build()`` always recompiles; ``ensure_built()`` compiles only
when the shared object is missing or older than its source.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_ref.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose=False):
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built():
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
