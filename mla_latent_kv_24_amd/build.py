"""Build the gfx950 MLA library (libmla.so) in-tree with hipcc.

    python -m mla_latent_kv_24_amd.build        # or __graft_entry__.build()

Every call compiles from source (objects in parallel, then one link).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla.so")
SOURCES = ["mla_api.hip", "mla_rope_absorb.hip", "mla_splitkv.hip", "mla_combine.hip", "mla_prefill.hip",
           "mla_gemm.hip", "mla_gemm_lds.hip", "mla_kvproj.hip", "mla_fp8.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the MLA library)")


def common_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # no packed-fp32 VALU forms anywhere in the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument"]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
