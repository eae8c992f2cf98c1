"""Build libfp8bq.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python fp8_blockwise_quantized_quantize_amd/build.py`` (this file
is self-contained: running it does not import the package, whose import
loads the library).  The library is written next to this file.
"""

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libfp8bq.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no fused multiply-add contraction beyond the explicit fmaf() calls:
    # the quantizer's quotient must be the exact IEEE one.
    "-ffp-contract=off",
    # MFMA results go to VGPRs (the per-K-block scale FMA reads them directly)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # packed FP32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build_library(verbose=False, extra_flags=()):
    """Compile every HIP source into LIB_PATH; raises CalledProcessError on failure."""
    srcs = sources()
    if not srcs:
        raise RuntimeError("no HIP sources under " + CSRC)
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line and "unknown target feature" not in line)
    if res.returncode != 0:
        sys.stderr.write(out + "\n")
        raise subprocess.CalledProcessError(res.returncode, cmd)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
