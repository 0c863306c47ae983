"""The C ABI from plain C: tests/c_abi_check.c (built by tests/c_abi_build.py,
which build() runs) drives libar.so with HIP runtime memory and a stream of
its own, and checks a sum, two fused calls and rejected calls against the
CPU oracle. It runs as a child process with a time limit."""
import os
import subprocess

import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "_build", "c_abi_check")


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_c_program_through_the_abi():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run __graft_entry__.build() (or tests/c_abi_build.py) first")
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and "c_abi_check: OK" in res.stdout, res.stdout + res.stderr
