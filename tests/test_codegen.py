"""Checks on the gfx950 code object of the libraries built here (no GPU).

The device code is unbundled from each library's .hip_fatbin section and
disassembled with the ROCm LLVM tools, then checked for:
  * no packed-fp32 arithmetic (the build turns the feature off; scalar fp32
    only);
  * no scalar-memory writes of any kind (stores, atomics, cache write-back or
    discard): every store goes through vector memory;
  * no register spills and no scratch (private segment) in any kernel;
  * the instructions the design relies on: 16-byte non-temporal vector loads
    and stores, and the packed round-to-nearest-even conversions to bf16 and
    fp16; in the streaming-ceiling library, both of its store forms
    (non-temporal global stores and device-scope buffer stores).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "tensor_all_reduce_ar_amd")
LLVM = "/opt/rocm/llvm/bin"
TOOLS = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump", "llvm-readelf")]
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

pytestmark = pytest.mark.skipif(not all(os.path.exists(t) for t in TOOLS), reason="ROCm LLVM tools not found")


def _code_object(lib, tmp_path):
    if not os.path.exists(lib):
        pytest.skip(f"{lib} not built")
    fatbin, dummy, co = tmp_path / "fatbin.bin", tmp_path / "host.so", tmp_path / "dev.co"
    subprocess.run([TOOLS[0], f"--dump-section=.hip_fatbin={fatbin}", lib, str(dummy)], check=True)
    subprocess.run([TOOLS[1], "--unbundle", "--type=o", f"--input={fatbin}", f"--targets={TARGET}",
                    f"--output={co}"], check=True)
    asm = subprocess.run([TOOLS[2], "-d", "--mcpu=gfx950", str(co)], check=True, capture_output=True,
                         text=True).stdout
    notes = subprocess.run([TOOLS[3], "--notes", str(co)], check=True, capture_output=True, text=True).stdout
    return asm, notes


def _mnemonics(asm):
    out = set()
    for line in asm.splitlines():
        m = re.match(r"\s+([a-z_][a-z0-9_]*)\b", line)
        if m:
            out.add(m.group(1))
    return out


@pytest.fixture(scope="module")
def libar(tmp_path_factory):
    return _code_object(os.path.join(PKG, "libar.so"), tmp_path_factory.mktemp("libar"))


@pytest.fixture(scope="module")
def libceiling(tmp_path_factory):
    return _code_object(os.path.join(PKG, "libstream_ceiling.so"), tmp_path_factory.mktemp("ceiling"))


SCALAR_WRITE = re.compile(r"^s_(buffer_)?(store|atomic)|^s_scratch_store|^s_dcache_(wb|discard)")
PACKED_FP32 = re.compile(r"^v_pk_(add|mul|fma)_f32$")


@pytest.mark.parametrize("which", ["libar", "libceiling"])
def test_no_packed_fp32_and_no_scalar_memory_writes(which, request):
    asm, _ = request.getfixturevalue(which)
    ops = _mnemonics(asm)
    assert ops, "empty disassembly"
    assert not sorted(o for o in ops if PACKED_FP32.match(o))
    assert not sorted(o for o in ops if SCALAR_WRITE.match(o))


@pytest.mark.parametrize("which", ["libar", "libceiling"])
def test_no_spills_and_no_scratch(which, request):
    _, notes = request.getfixturevalue(which)
    for key in ("vgpr_spill_count", "sgpr_spill_count", "private_segment_fixed_size"):
        values = re.findall(rf"\.{key}:\s+(\d+)", notes)
        assert values, key
        assert set(values) == {"0"}, (key, sorted(set(values)))


def test_vector_path_instructions(libar):
    asm, _ = libar
    assert re.search(r"global_load_dwordx4 .* nt", asm), "16-byte non-temporal loads"
    assert re.search(r"global_store_dwordx4 .* nt", asm), "16-byte non-temporal stores"
    ops = _mnemonics(asm)
    assert "v_cvt_pk_bf16_f32" in ops, "packed RNE conversion to bf16"
    assert "v_cvt_pk_f16_f32" in ops, "packed RNE conversion to fp16"


def test_ceiling_load_and_store_forms(libceiling):
    asm, _ = libceiling
    assert re.search(r"global_load_dwordx4 .* nt", asm), "16-byte non-temporal global loads"
    bl = re.findall(r"buffer_load_dwordx4 .*", asm)
    assert bl, "16-byte buffer loads"
    assert all(re.search(r"\bnt\b", x) and not re.search(r"\b(sc0|sc1)\b", x) for x in bl), bl[:3]
    assert re.search(r"global_store_dwordx4 .* nt", asm), "16-byte non-temporal global stores"
    sc1 = re.findall(r"buffer_store_dwordx4 .*", asm)
    assert sc1, "16-byte buffer stores"
    assert all(re.search(r"\bsc1\b", x) and not re.search(r"\b(nt|sc0)\b", x) for x in sc1), sc1[:3]


def test_row_sums_reduce_through_dpp_not_lds_permutes(libar):
    """The wave-level sum of squares moves lanes with DPP (pair and quad
    swaps, row mirrors, the row broadcasts 15 and 31) and reads the total back
    with v_readlane; no ds_bpermute (an LDS round trip per step) is left."""
    asm, _ = libar
    ops = _mnemonics(asm)
    assert "ds_bpermute_b32" not in ops
    for ctrl in (r"quad_perm:\[1,0,3,2\]", r"quad_perm:\[2,3,0,1\]", r"row_half_mirror", r"row_mirror",
                 r"row_bcast:15 row_mask:0xa", r"row_bcast:31 row_mask:0xc"):
        assert re.search(r"_dpp .*" + ctrl, asm), ctrl
    assert "v_readlane_b32" in ops
