"""Build libflashattn.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libflashattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip", "fa_quant.hip", "fa_fwd8.hip", "fa_fwd32.hip"]
# Packed fp32 VALU ops are switched off on purpose: every fp32 op stays a plain
# v_*_f32 instruction.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]
# Per-source extra flags: MFMA accumulators in VGPRs, so that the softmax and
# gradient VALU work reads the scores without copies out of AGPRs (AGPRs then
# serve as extra storage for long-lived values).
SOURCE_FLAGS = {
    "fa_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "fa_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "fa_fwd8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
