"""Builds libpagedkv.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libpagedkv.so")
SOURCES = ["api.hip", "store.hip", "decode.hip", "prefill.hip", "measure.hip", "block_manager.cpp"]
ARCH = "gfx950"

# Packed-FP32 instructions are disabled for the device code: hipcc would otherwise form them from
# plain float code.
HIPCC_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", CSRC, "-I", INCLUDE]


# prefill: softmax maxima over MFMA results need no NaN quieting (masked scores are -inf, never NaN),
# so IEEE mode is off there and fmax is a single v_max_f32.
# measure: MFMA accumulators in VGPRs; the default form there keeps them in AGPRs and copies every chain
# through VGPRs on each loop turn, which would understate the matrix cores' issue rate.
FILE_FLAGS = {"prefill.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
              "measure.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source to an object, then link the shared library. Always recompiles."""
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        if verbose:
            print(" ".join(cmd))
        return obj

    with ThreadPoolExecutor(min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
