"""The C ABI from plain C: tests/c_abi_check.c (built by tests/c_abi_build.py,
which build() runs) drives libar.so with HIP runtime memory and a stream of
its own, and checks against the CPU oracle a sum, two fused calls, rejected
calls, the two-shot slices of both ops, the unfused path and a sum replayed
from a HIP graph. It runs as a child process with a time limit."""
import os
import re
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

    def count(prefix):
        return sum(line.startswith(prefix) for line in log)

    for prefix in ("[ar] sum pack R=3 V=8 n=10007 ", "[ar] fused pack R=4 rows=37 H=640 ppr=80 ",
                   "[ar] fused pack R=2 rows=9 H=1024 ppr=256 ", "[ar] sum pack R=8 V=8 n=65536 ",
                   "[ar] fused pack R=1 rows=16 H=4096 ppr=512 ", "[ar] sum pack R=2 V=8 n=1000003 "):
        assert count(prefix) == 1, (prefix, log)
    # the slices: 3 sums that share 10007 elements, 4 fused calls that share 37 rows
    sliced = [int(m.group(1)) for m in (re.match(r"\[ar\] sum pack R=4 V=8 n=(\d+) ", x) for x in log) if m]
    assert sorted(sliced) == [3335, 3336, 3336], log
    rows = [int(m.group(1)) for m in (re.match(r"\[ar\] fused pack R=3 rows=(\d+) H=1536 ", x) for x in log) if m]
    assert sorted(rows) == [7, 10, 10, 10], log
    # one line per launched call; the graph's replays launch from the graph, not through the library
    assert len(log) == 13, log
