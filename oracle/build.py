"""Compile the FP64 reference attention (test infrastructure) with gcc.

The oracle is plain C built by the host compiler (``-O3 -march=native
-fopenmp``); it shares nothing with the GPU library.  ``-march=native``
targets the CPU that builds it, so the build records that CPU (model name
and feature flags) beside the shared object, and ``ensure_built()``
recompiles on a host whose CPU differs (a benchmark host is not the build
host).  ``-std=c11`` keeps floating-point contraction off, so the arithmetic
is the same on every host.  ``build()`` always recompiles.
"""
import hashlib
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_ref.c")
LIB = os.path.join(HERE, "liboracle.so")
HOST_TAG = os.path.join(HERE, "liboracle.host")
FLAGS = ["-O3", "-march=native", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]


def host_signature():
    """Model name and feature flags of this host's first CPU, hashed."""
    keep = []
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break
                if line.startswith(("model name", "flags", "vendor_id")):
                    keep.append(line.strip())
    except OSError:
        pass
    return hashlib.sha256("\n".join(keep).encode()).hexdigest()[:16]


def build(verbose=False):
    cmd = ["gcc"] + FLAGS + ["-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    with open(HOST_TAG + ".tmp", "w") as f:
        f.write(host_signature() + "\n")
    os.replace(HOST_TAG + ".tmp", HOST_TAG)
    return LIB


def _built_for_this_host():
    try:
        with open(HOST_TAG) as f:
            return f.read().strip() == host_signature()
    except OSError:
        return False


def ensure_built():
    if (not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC)
            or not _built_for_this_host()):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
