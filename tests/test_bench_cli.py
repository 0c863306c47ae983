"""The benchmark's command line on a host (no GPU needed): more than one GPU
is refused with an explanation before any GPU work, whether asked for with
--gpus or by a multi-process launcher's WORLD_SIZE."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    res = _run(["--gpus", "2"])
    assert res.returncode == 2, res.stderr
    assert "one GPU only" in res.stderr
    assert res.stdout == ""


def test_multi_process_launch_is_refused():
    res = _run([], {"WORLD_SIZE": "4"})
    assert res.returncode == 2, res.stderr
    assert "--gpus 4 is not supported" in res.stderr
