"""Build libtriattn.so (gfx950) in-tree with hipcc.

Usage: ``python -m masked_attention_tri_amd.build``.  Every call recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtriattn.so")
SOURCES = ["triattn_api.hip", "kernel_generic.hip", "kernel_mfma.hip", "kernel_mfma_d32.hip",
           "kernel_mfma_d64.hip", "kernel_mfma_d128.hip", "kernel_mfma_d256.hip",
           "kernel_util.hip", "kernel_bwd.hip", "kernel_bwd_d32.hip", "kernel_bwd_d64.hip",
           "kernel_bwd_d128.hip", "noalloc.hip", "kernel_fp32.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 instructions are disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs: the softmax reads and rescales them
    # with VALU instructions, and AGPR accumulators cost a copy each way
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall",
    "-Wno-unused-function",
    f"-I{INCLUDE}",
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature;
    # that line is expected noise.
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    return res.returncode, msgs


def build(verbose: bool = False, extra_flags=None, jobs: int = 0) -> str:
    """Compile every HIP source into one shared library; return its path.

    The sources compile to objects in parallel (up to `jobs` at once, default
    min(8, CPUs)), then link; every call recompiles."""
    from concurrent.futures import ThreadPoolExecutor

    jobs = jobs or min(8, os.cpu_count() or 1)
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"] + list(extra_flags or [])
    cmds = [[HIPCC, *compile_flags, "-c", "-o", os.path.join(objdir, src + ".o"),
             os.path.join(CSRC, src)] for src in SOURCES]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        results = list(pool.map(_run, cmds))
    for (rc, msgs), src in zip(results, SOURCES):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
        if verbose and msgs:
            print("\n".join(msgs))
    out_tmp = LIB + ".tmp"
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp,
            *[os.path.join(objdir, src + ".o") for src in SOURCES]]
    rc, msgs = _run(link)
    if rc != 0:
        raise RuntimeError("link failed:\n" + "\n".join(msgs))
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
