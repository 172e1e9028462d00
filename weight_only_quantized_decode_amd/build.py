"""Build libwqd.so in-tree with hipcc for gfx950 (no JIT cache, nothing installed).

    python -m weight_only_quantized_decode_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libwqd.so")
SOURCES = ["wqd_plan.cpp", "wqd_api.cpp", "wqd_pack.hip", "wqd_gemv.hip", "wqd_gemv_bcast.hip", "wqd_gemv_mc.hip", "wqd_skinny.hip", "wqd_gemm.hip", "wqd_gemm_lds.hip", "wqd_mfma.hip", "wqd_stream.hip", "wqd_spec.hip", "wqd_noalloc.hip", "wqd_w8a8.hip", "wqd_attn.hip", "wqd_chain.hip"]
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}"]
# Keep the compiler from forming packed-FP32 (v_pk_*_f32) instructions.
NO_PACKED_F32 = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-file flags: the tiled matrix-core kernel keeps its accumulators in VGPRs
# (in AGPRs the compiler copied them at every loop edge, and the 4-wavefront
# instances needed over 256 registers).
EXTRA = {"wqd_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "wqd_gemm_lds.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "wqd_w8a8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         # decode attention: 234 registers in VGPR form (two wavefronts per SIMD) against 272 with AGPRs
         "wqd_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *NO_PACKED_F32, *EXTRA.get(src, []), "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
