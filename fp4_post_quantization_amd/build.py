"""Build libfp4q.so (the C-ABI library) for gfx950 with hipcc, in place."""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libfp4q.so")
SOURCES = [os.path.join(PKG, "csrc", "fp4q.hip"), os.path.join(PKG, "csrc", "fp4q_gemm.hip")]
HEADERS = [os.path.join(PKG, "csrc", "fp4q_device.h"), os.path.join(ROOT, "include", "fp4q.h"),
           os.path.join(ROOT, "include", "fp4q_gemm.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # bit-exact float32 arithmetic: no contraction into FMA, IEEE division
    # and denormals (the HIP defaults) are kept
    "-ffp-contract=off",
    # no packed-FP32 VALU instructions in any generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose=False):
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libfp4q.so")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
