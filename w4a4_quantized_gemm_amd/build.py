"""Build libsvdq.so in-tree for gfx950 with hipcc.

    python -m w4a4_quantized_gemm_amd.build        # or build() from Python

HIP sources (*.hip) are compiled by hipcc for gfx950 only; the HIP-free host
sources (*.cpp: validation, blob layout, the small eigensolver) by g++.
Objects go to w4a4_quantized_gemm_amd/_build/, the shared library to
w4a4_quantized_gemm_amd/libsvdq.so; the peak-measurement probes
(csrc_peaks/, include/svdq_peaks.h) to libsvdq_peaks.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsvdq.so")
PEAKS_LIB = os.path.join(PKG, "libsvdq_peaks.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall"]
# packed fp32 VALU ops are disabled for every device compilation
# private arrays stay in registers/scratch rather than being promoted into
# LDS, which the GEMM kernels size and use themselves
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fno-gpu-rdc", "-ffp-contract=off", "-mllvm", "-disable-promote-alloca-to-lds"]


# per-file device flags: the INT4 GEMM dequantizes each group's MFMA result
# with VALU code, so its MFMAs write VGPRs directly (otherwise every result
# would be read out of the accumulation registers first)
FILE_FLAGS = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        extra = FILE_FLAGS.get(os.path.basename(src), [])
        cmd = [HIPCC, *HIP_FLAGS, *extra, *COMMON, "-x", "hip", "-c", src, "-o", obj]
    else:
        cmd = ["g++", *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass reports the device-only feature flag as unknown: harmless
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(verbose: bool = True, jobs: int = 8) -> str:
    """Compile every source and link libsvdq.so; returns the library path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-lquadmath"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, LIB)
    # the peak-measurement probes (a measurement aid, a library of its own)
    pobj = _compile(os.path.join(PKG, "csrc_peaks", "peaks.hip"))
    ptmp = PEAKS_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", ptmp, pobj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(ptmp, PEAKS_LIB)
    if verbose:
        print(f"built {LIB} and {PEAKS_LIB}")
    return LIB


if __name__ == "__main__":
    build()
