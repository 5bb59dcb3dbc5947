"""Build libmla.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m mla_latent_kv_03_amd.build      # or __graft_entry__.build()

The library lands next to this file, so the Python binding finds it and a
copy of the tree carries it. Every HIP source is compiled with the packed-fp32
target feature turned off (the compiler is then never allowed to emit packed
fp32 adds/multiplies/FMAs).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla.so")
ARCH = "gfx950"

SOURCES = ["mla_api.cpp", "mla_kernels.hip", "mla_decode_rows16.hip", "mla_decode_ws.hip",
           "mla_proj_mfma.hip", "mla_q8.hip", "mla_sparse.hip", "mla_prefill.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wshadow", "-Wno-unused-function", "-fvisibility=hidden",
    # keep MFMA accumulators in ordinary VGPRs: the online softmax rescales
    # them with vector ALU ops, which cannot address the accumulation registers
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmla")


def build(verbose: bool = False) -> str:
    """Compile every source and link libmla.so; returns the library path."""
    cc = hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, src + ".o")
        cmd = [cc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", path, "-o", obj]
        if src.endswith(".cpp"):
            cmd = [cc, "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
                   "-I", os.path.join(ROOT, "include"),
                   "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
