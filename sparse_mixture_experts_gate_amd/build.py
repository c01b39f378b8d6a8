"""Builds libdsmoe.so in-tree for gfx950 with hipcc (one object per source,
compiled in parallel, then linked)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsmoe.so")
# achievable-peak microbenchmarks for bench.py, a library of their own
MB_LIB = os.path.join(PKG, "libdsmoe_microbench.so")
MB_SOURCE = "microbench.hip"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep the compiler from emitting packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]
# routing and quantization decide integers from fp32 values: no contraction
NO_CONTRACT = {"router.hip", "elementwise.hip", "balance.hip", "backward_fp8.hip"}
# MFMA results in VGPRs: the FP8 kernels scale every product on the VALU, and
# with the product in AGPRs the compiler reused one AGPR quad per product,
# which serialized the MFMAs of the decode tiles behind the copies out
MFMA_VGPR = {"gemm_fp8.hip", "backward_fp8.hip"}
SOURCES = ["dsmoe_api.cpp", "router.hip", "permute.hip", "gemm_bf16.hip", "gemm_f32.hip",
           "gemm_fp8.hip", "elementwise.hip", "backward.hip", "balance.hip", "backward_fp8.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *COMMON]
    if src in NO_CONTRACT:
        cmd.append("-ffp-contract=off")
    if src in MFMA_VGPR:
        cmd += ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + [MB_SOURCE]
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:-1], LIB)
    _link(objs[-1:], MB_LIB)
    if verbose:
        print(f"built {LIB} and {MB_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
