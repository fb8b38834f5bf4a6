"""Build tests/c_abi/abi_check: a plain C program (gcc, C11) that drives the
attention library through include/fa.h and checks it against the FP64 oracle.

It links io_aware_exact_03_amd/libfa.so, oracle/liboracle.so and the HIP
runtime, with run paths relative to the binary, so both libraries must be
built first (``python __graft_entry__.py build`` builds all three).
``build()`` always recompiles.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_check.c")
EXE = os.path.join(HERE, "abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose=False):
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           SRC, "-o", EXE + ".tmp",
           "-L", os.path.join(ROOT, "io_aware_exact_03_amd"), "-lfa",
           "-L", os.path.join(ROOT, "oracle"), "-loracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../io_aware_exact_03_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
