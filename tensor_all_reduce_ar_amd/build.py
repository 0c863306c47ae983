"""Build the C-ABI libraries of HIP kernels for gfx950, in-tree.

    python -m tensor_all_reduce_ar_amd.build

``libar.so`` (csrc/ar.hip, include/ar.h) is the all-reduce core;
``libstream_ceiling.so`` (csrc/stream_ceiling.hip, include/stream_ceiling.h)
holds the streaming-ceiling kernels the benchmark times beside it. hipcc
cross-compiles without a GPU. Extra ``-D`` definitions (tuning macros of
csrc/ar.hip) can be passed through ``build(defines=...)``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from typing import Dict, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "ar.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libar.so")
CEILING_SRC = os.path.join(PKG, "csrc", "stream_ceiling.hip")
CEILING_LIB = os.path.join(PKG, "libstream_ceiling.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions in device code (scalar fp32 arithmetic only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _compile(src: str, out: str, defines: Optional[Dict[str, int]], verbose: bool) -> str:
    cmd = [HIPCC, *HIPCC_FLAGS, "-I", INCLUDE]
    for k, v in (defines or {}).items():
        cmd.append(f"-D{k}={v}")
    tmp = out + ".tmp%d" % os.getpid()
    cmd += ["-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(out: Optional[str] = None, defines: Optional[Dict[str, int]] = None, verbose: bool = False) -> str:
    """Build libar.so (or `out`) from csrc/ar.hip."""
    return _compile(SRC, out or LIB, defines, verbose)


def build_ceiling(verbose: bool = False) -> str:
    """Build libstream_ceiling.so from csrc/stream_ceiling.hip."""
    return _compile(CEILING_SRC, CEILING_LIB, None, verbose)


def build_all(verbose: bool = False) -> None:
    build(verbose=verbose)
    build_ceiling(verbose=verbose)


if __name__ == "__main__":
    build_all(verbose=True)
    sys.exit(0)
