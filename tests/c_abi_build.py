"""Build the plain-C check of the C ABI (tests/c_abi_check.c) on the host:

    python tests/c_abi_build.py

gcc compiles it together with the CPU oracle (oracle/ar_oracle.c, with the
oracle's own floating-point flags) and links libar.so and the HIP runtime;
the binary is tests/_build/c_abi_check. No GPU is needed to build it;
tests/test_gpu_c_abi.py runs it on one.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "tensor_all_reduce_ar_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
EXE = os.path.join(HERE, "_build", "c_abi_check")


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    tmp = EXE + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           "-o", tmp, os.path.join(HERE, "c_abi_check.c"), os.path.join(ROOT, "oracle", "ar_oracle.c"),
           "-L", PKG, "-lar", "-Wl,-rpath,$ORIGIN/../../tensor_all_reduce_ar_amd",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
