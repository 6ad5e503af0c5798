"""Build libtc.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m linear_attention_tensor_amd.build

Compiles every source under ``csrc/`` with hipcc, links
``linear_attention_tensor_amd/libtc.so`` and replaces the old library
atomically.  Needs no GPU (hipcc cross-compiles).
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtc.so")

SOURCES = ["tc_api.cpp", "tc_scan.hip", "tc_decode.hip", "tc_fused.hip", "tc_swa.hip", "tc_window.hip", "tc_window_bwd.hip", "tc_window_bwd_mfma.hip", "tc_convert.hip", "delta_scan.hip", "delta_bf16.hip",
           "delta_bwd.hip", "tc_memory.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    f"--offload-arch={ARCH}",
    # no packed fp32 instructions: their results are not trusted on these parts
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
]


# Sources whose kernels keep their MFMA accumulators in VGPRs: without the
# option the compiler places them in AGPRs and copies them back to VGPRs in
# the hot loops (about 60 extra VALU moves per chunk in the delta-rule walk);
# with it those kernels need fewer registers, spill nothing and run 1-2 %
# faster (same-box A/B of the benchmark).  The window main kernel and the
# decode kernels never used AGPRs and keep the plain build.
VGPR_FORM = {"tc_fused.hip", "tc_scan.hip", "tc_window_bwd_mfma.hip", "delta_bwd.hip", "tc_memory.hip",
             "delta_bf16.hip"}


def _compile(src: str) -> str:
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", out]
    if src in VGPR_FORM:
        cmd += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return out


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
