"""The library driven from plain C (tests/c_abi/abi_check.c) through
include/fa.h alone, as a C caller would use it: argument checks on the CPU,
and on the GPU forward (bf16 with causal, key-padding and block masks; fp32)
and backward calls on a caller-created stream compared with the FP64
oracle.  The program is built by ``__graft_entry__.build()``
(tests/c_abi/build.py) and runs as a child process."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi", "abi_check")


def _exe():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built; run `python __graft_entry__.py build`")
    return EXE


def _run(args, timeout):
    r = subprocess.run([_exe()] + args, capture_output=True, text=True, timeout=timeout)
    sys.stdout.write(r.stdout)
    return r


def test_c_abi_argument_checks():
    r = _run(["--errors-only"], 60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all cases passed" in r.stdout


@pytest.mark.gpu
def test_c_abi_on_gpu():
    r = _run([], 120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all cases passed" in r.stdout
    assert r.stdout.count("max|dO|") == 4 and r.stdout.count("max err") == 3
