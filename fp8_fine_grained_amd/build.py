"""Build libfp8fg.so (all HIP sources, gfx950 only) in the package directory."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfp8fg.so")
SOURCES = ["api.hip", "quant.hip", "gemm.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no hand-written or compiler-generated packed FP32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division for the quantizers; no fast-math anywhere
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    # MFMA results straight into arch VGPRs: the per-K-block promotion FMAs
    # read them without v_accvgpr_read round trips
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def build(verbose=False):
    """Compile every HIP source into one shared library; raises on failure."""
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include")] + \
          [os.path.join(CSRC, s) for s in SOURCES] + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libfp8fg.so")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
