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


# Host-code sanitizers (AddressSanitizer, UndefinedBehaviorSanitizer) for a
# checking build: each flag applies to the host pass only, the device code is
# compiled as usual.  The result needs the sanitizer runtime preloaded, e.g.
#   LD_PRELOAD=$(/opt/rocm/bin/hipcc -print-file-name=libclang_rt.asan-x86_64.so)
HOST_SANITIZE = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan"]


def build(verbose=False, out=None, host_sanitize=False):
    """Compile libfp4q.so in place (or to ``out``); host_sanitize builds the
    checking variant described above, which must not replace the library."""
    target = out or LIB
    if host_sanitize and os.path.abspath(target) == LIB:
        raise ValueError("the host-sanitized build goes to a path of its own")
    flags = FLAGS + (HOST_SANITIZE if host_sanitize else [])
    cmd = [HIPCC, *flags, "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", target + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building " + target)
    os.replace(target + ".tmp", target)
    return target


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--host-sanitize", metavar="OUT", help="build the host-sanitized checking library at OUT")
    a = ap.parse_args()
    print(build(verbose=True, out=a.host_sanitize, host_sanitize=bool(a.host_sanitize)))
