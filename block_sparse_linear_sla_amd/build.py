"""Build libsla.so (the HIP kernels and the C interface) for gfx950 with hipcc.

Usage: python -m block_sparse_linear_sla_amd.build [-v]
The shared library is written next to this file; objects go to _build/.
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
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsla.so")
SOURCES = ["sla_api.hip", "mask.hip", "attn_bf16.hip", "attn_f32.hip", "attn_i8.hip", "attn_bwd.hip", "attn_bwd_lin.hip"]
# per-source extra flags: the attention kernels keep their matrix accumulators
# in ordinary VGPRs (their softmax reads them every step), so the compiler is
# told to use the VGPR form of the MFMA instructions there.  The 8-bit file
# decides integer codes from float32 expressions that must round exactly as
# written, so it is built without floating-point contraction.
EXTRA = {"attn_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "attn_bwd_lin.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "attn_i8.hip": ["-ffp-contract=off", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
ARCH = os.environ.get("SLA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # packed fp32 vector ops stay off: the compiler must not emit them
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-result", "-Wno-pass-failed", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *flags(), *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libsla.so; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
