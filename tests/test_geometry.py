"""Host check of the fused op's launch geometry (csrc/fused_geometry.h, the
header the library's dispatch uses) for every row width of 1..8192 packs:
tests/geometry_check.cpp, built with the host C++ compiler and run here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tensor_all_reduce_ar_amd", "csrc")
CHECK = os.path.join(ROOT, "tests", "geometry_check.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_every_row_width_has_a_valid_launch_shape(tmp_path):
    exe = tmp_path / "geometry_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC, "-o", str(exe), CHECK], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().startswith("ok ")
    assert int(res.stdout.split()[1]) > 8192 * 4
