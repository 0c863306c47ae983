"""Build ``libar.so`` (the C-ABI library of HIP kernels) for gfx950, in-tree.

    python -m tensor_all_reduce_ar_amd.build

hipcc cross-compiles without a GPU. Extra ``-D`` definitions (tuning macros of
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
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions in device code (scalar fp32 arithmetic only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(out: Optional[str] = None, defines: Optional[Dict[str, int]] = None, verbose: bool = False) -> str:
    out = out or LIB
    cmd = [HIPCC, *HIPCC_FLAGS, "-I", INCLUDE]
    for k, v in (defines or {}).items():
        cmd.append(f"-D{k}={v}")
    tmp = out + ".tmp%d" % os.getpid()
    cmd += ["-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
