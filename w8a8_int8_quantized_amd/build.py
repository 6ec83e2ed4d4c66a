"""Build libw8a8.so in-tree with hipcc for gfx950.

    python w8a8_int8_quantized_amd/build.py     (a plain script: it does not
                                                 import the package, which
                                                 needs the built library)

Every HIP source under csrc/ is compiled to an object, then linked into
w8a8_int8_quantized_amd/libw8a8.so.  Flags:
  -O3 --offload-arch=gfx950           CDNA4 only, no other targets
  -ffp-contract=off                   no silent mul+add fusion: the quantiser's
                                      fp32 steps must round exactly as written
  -fhip-fp32-correctly-rounded-divide-sqrt
                                      IEEE fp32 division for scale = amax / 127
                                      and the exact-quotient path
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                      no packed-fp32 VALU instructions
  -mllvm -amdgpu-mfma-vgpr-form       gemm_block.hip only: MFMA results in
                                      VGPRs, where the dequantising VALU
                                      reads them (the channel kernel keeps its
                                      256 accumulators per lane in AGPRs)
"""

import os
import subprocess
import sys
import concurrent.futures as cf

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libw8a8.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["quant.hip", "gemm_tile.hip", "gemm_block.hip", "gemm_decode.hip", "asym.hip", "capi.cpp"]
EXTRA_FLAGS = {"gemm_block.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    "--offload-arch=gfx950",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON_FLAGS + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + COMMON_FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
