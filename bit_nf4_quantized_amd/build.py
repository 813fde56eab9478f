"""Build the HIP library libqlora_nf4.so in-tree for gfx950 with hipcc.

Every source is compiled (in parallel) to an object and linked into one
shared library next to this file. Flags that the numerics depend on:
  -ffp-contract=off                       no fused multiply-add contraction,
                                          so each fp32 step rounds once
  -fhip-fp32-correctly-rounded-divide-sqrt  IEEE fp32 division
  -fno-gpu-flush-denormals-to-zero        IEEE gradual underflow
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed fp32 VALU ops
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libqlora_nf4.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
OBJ_DIR = os.path.join(ROOT, "_build")
SOURCES = ["api.cpp", "quantize.hip", "gemm.hip", "gemv.hip", "gemv1.hip", "dense_gemm.hip", "skinny_gemm.hip", "int8.hip", "merge.hip", "midm.hip", "dropout.hip", "optim.hip", "convcheck.hip", "probe.hip"]
ARCH = os.environ.get("QLORA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-fno-gpu-flush-denormals-to-zero",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
    ]


# Per-source code-generation options: the GEMV kernels keep MFMA results in
# VGPRs (their accumulators feed VALU FMAs; AGPR copies would cost VALU issue).
EXTRA_FLAGS = {"gemv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, src + ".o")
    cmd = [hipcc()] + common_flags() + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
