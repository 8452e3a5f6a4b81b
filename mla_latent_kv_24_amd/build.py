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
           "mla_gemm.hip", "mla_gemm_lds.hip", "mla_kvproj.hip", "mla_fp8.hip",
           "mla_probe.hip"]
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


PROBE_LIB = os.path.join(PKG, "libmla_probe.so")


def build(verbose: bool = False, probe: bool = False) -> str:
    """Compile and link libmla.so; with probe=True, libmla_probe.so instead:
    the same library with per-phase cycle stamps in the 128-head decode
    kernel and the read, LDS and MFMA probe kernels of mla_probe.hip
    (MLA_PHASE_STAMPS, driven by probe.py), a measurement build that the
    product never loads."""
    cc = hipcc()
    objdir = os.path.join(PKG, "_build_probe" if probe else "_build")
    os.makedirs(objdir, exist_ok=True)
    extra = ["-DMLA_PHASE_STAMPS"] if probe else []
    out_lib = PROBE_LIB if probe else LIB

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *common_flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out_lib + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out_lib)
    return out_lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, probe="--probe" in sys.argv))
