"""Build libkvq.so in-tree with hipcc for gfx950.

    python -m quantized_decode_attention_03_amd.build

Every HIP source under csrc/ is compiled into one shared library next to this
file. Flags: correctly rounded fp32 division (the quantizer's divisions must be
IEEE), no fast-math, packed-fp32 instructions disabled, and MFMA
accumulators kept in VGPRs.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libkvq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # MFMA accumulators in ordinary VGPRs (no AGPR copies around each MFMA)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose=True):
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"),
                             "-I", os.path.join(HERE, "csrc"), "-o", tmp] + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
