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


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_dispatch_log():
    """AR_LOG=1 (read once per process) prints each dispatch decision to
    stderr: kernel, shape and launch geometry of every call the C check
    makes, and nothing for the calls it expects to be rejected."""
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run __graft_entry__.build() (or tests/c_abi_build.py) first")
    env = dict(os.environ, AR_LOG="1")
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 0 and "c_abi_check: OK" in res.stdout, res.stdout + res.stderr
    log = [line for line in res.stderr.splitlines() if line.startswith("[ar] ")]
    assert any(line.startswith("[ar] sum pack R=3 V=8 n=10007 ") for line in log), log
    assert any(line.startswith("[ar] fused pack R=4 rows=37 H=640 ppr=80 ") for line in log), log
    assert any(line.startswith("[ar] fused pack R=2 rows=9 H=1024 ppr=256 ") for line in log), log
    assert len(log) == 3, log
