"""Build the gfx950 library libhts.so in-tree with hipcc (no JIT, no torch extension).

Usage: python -m tile_gemm_amd.build   (or tile_gemm_amd.build.build())
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhts.so")
# measured roofline denominators (streaming read, register-operand matrix-core throughput)
PEAK_LIB = os.path.join(PKG, "libhts_peak.so")
PEAK_SOURCES = ["peak.hip"]
OBJDIR = os.path.join(ROOT, "_build")

SOURCES = ["hts_api.cpp", "pack.hip", "gemm_decode.hip", "gemm_prefill.hip", "wanda.hip", "elementwise.hip"]

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms stay off; plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no contraction of separate multiplies and adds: bit-exact selection and sums
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# matrix-core accumulators in VGPRs: dense and sparse instructions then share them without
# AGPR<->VGPR copies at the type branches (the AGPR file still takes register spills)
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libhts.so)")


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    # every source, the host API included, is compiled as HIP (it calls the HIP runtime)
    cmd = [hipcc(), *COMMON, *VGPR_FORM, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + PEAK_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PEAK_SOURCES], PEAK_LIB)
    if verbose:
        print(f"built {LIB} and {PEAK_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
