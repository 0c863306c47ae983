"""The streaming-ceiling library (measurement only): exports, host-side
argument checks (no GPU), and on the GPU that every output is the XOR of the
inputs over sizes with and without a partial last step."""
import os
import re
import subprocess

import numpy as np
import pytest

from tensor_all_reduce_ar_amd import stream_ceiling as sc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "stream_ceiling.h")
A = 0x7F0000000000  # made-up aligned addresses: every call below is rejected before use


def test_library_exports_the_declared_function():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    declared = re.findall(r"^\s*[a-z_0-9]+\s+(sc_[a-z_0-9]+)\s*\(", text, flags=re.M)
    assert declared == ["sc_stream"]
    sc.load()
    nm = subprocess.run(["nm", "-D", "--defined-only", sc.LIB_PATH], capture_output=True, text=True, check=True)
    assert "sc_stream" in re.findall(r"\bT (sc_\w+)", nm.stdout)


@pytest.mark.parametrize("n_in,n_out", [(0, 1), (13, 0), (1, 3)])
def test_bad_counts(n_in, n_out):
    assert sc.sc_stream_raw([A] * n_in, [A + 4096] * n_out, 1024) == -1


def test_negative_counts():
    import ctypes
    ins = (ctypes.c_void_p * 2)(A, A + 4096)
    outs = (ctypes.c_void_p * 1)(A + 8192)
    assert sc.load().sc_stream(ins, 2, outs, -1, 1024, 0, None) == -1
    assert sc.load().sc_stream(ins, -2, outs, 1, 1024, 0, None) == -1


@pytest.mark.parametrize("shape", [-1, 16])
def test_bad_shape(shape):
    assert sc.sc_stream_raw([A], [A + 4096], 1024, shape) == -4


def test_null_and_alignment():
    assert sc.sc_stream_raw([A, 0], [A + 4096], 1024) == -2
    assert sc.sc_stream_raw([A], [0], 1024) == -2
    assert sc.sc_stream_raw([A + 8], [A + 4096], 1024) == -3
    assert sc.sc_stream_raw([A], [A + 4104], 1024) == -3
    assert sc.sc_stream_raw([A], [A + 4096], 1000) == -3


def test_zero_bytes_is_a_noop_without_any_hip_call():
    assert sc.sc_stream_raw([A, A + 4096], [A + 8192], 0) == 0


@pytest.mark.gpu
@pytest.mark.parametrize("shape", sorted(sc.SHAPES))
@pytest.mark.parametrize("n_in,n_out", [(1, 0), (1, 1), (4, 1), (9, 2), (12, 2)])
def test_outputs_are_the_xor_of_the_inputs(n_in, n_out, shape):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    rng = np.random.default_rng(n_in * 10 + n_out)
    for packs in (1, 1023, 1024, 2048, 3 * 2048 + 5, 100003):
        print(f"[stream] n_in={n_in} n_out={n_out} shape={shape} packs={packs}", flush=True)
        host = [rng.integers(0, 2 ** 32, size=4 * packs, dtype=np.uint32) for _ in range(n_in)]
        ins = [torch.from_numpy(h.view(np.int32)).cuda() for h in host]
        guard = 1024
        raw = [torch.full((4 * packs + 2 * guard,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
               for _ in range(n_out)]
        outs = [r[guard:guard + 4 * packs] for r in raw]
        sc.sc_stream(ins, outs, shape)
        torch.cuda.synchronize()
        want = np.bitwise_xor.reduce(np.stack(host), axis=0)
        for r in raw:
            b = r.cpu().numpy().view(np.uint32)
            assert np.array_equal(b[guard:guard + 4 * packs], want)
            assert np.all(b[:guard] == 0x5A5A5A5A) and np.all(b[guard + 4 * packs:] == 0x5A5A5A5A)
