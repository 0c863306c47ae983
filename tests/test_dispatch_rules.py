"""The C ABI's host rules (csrc/dispatch_rules.h: validation, vector-path
choice, two-shot slices, partials layout) and the fused launch geometry
(csrc/fused_geometry.h) under AddressSanitizer and UndefinedBehaviorSanitizer,
unsigned-integer overflow included: tests/dispatch_rules_check.cpp is built
with clang++ and run here. It drives fixed overflow cases (byte counts that
wrap size_t, buffers past the end of the address space, layouts that do not
fit) and 400k random adversarial parameter blocks, checking the invariants
every accepted call must keep. Host only: no pointer is ever dereferenced."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tensor_all_reduce_ar_amd", "csrc")
CHECK = os.path.join(ROOT, "tests", "dispatch_rules_check.cpp")
CLANG = next((c for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")) if c and os.path.exists(c)), None)
SAN = "-fsanitize=address,undefined,unsigned-integer-overflow"


def _build(tmp_path, flags):
    exe = tmp_path / "dispatch_rules_check"
    cmd = [CLANG, "-std=c++17", "-O1", "-g", *flags, "-fno-omit-frame-pointer", "-Wall", "-Werror",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", str(exe), CHECK]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


@pytest.mark.skipif(CLANG is None, reason="needs clang++ with the sanitizer runtimes")
def test_host_rules_clean_under_sanitizers(tmp_path):
    exe = _build(tmp_path, [SAN, "-fno-sanitize-recover=all"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-2000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-2000:]
    assert r.stdout.startswith("ok ") and int(r.stdout.split()[1]) > 1_000_000, r.stdout


@pytest.mark.skipif(CLANG is None, reason="needs clang++")
def test_host_rules_unsanitized_build_agrees(tmp_path):
    """The same checks in an optimised build without sanitizers (the code the
    library ships is built at -O3)."""
    exe = _build(tmp_path, ["-O3"])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok "), (r.stdout[-2000:], r.stderr[-2000:])
