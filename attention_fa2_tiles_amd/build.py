"""Build libfa2tiles.so (gfx950) in-tree with hipcc.

    python -m attention_fa2_tiles_amd.build        # or: python attention_fa2_tiles_amd/build.py

Each source is compiled to an object under ``_build/`` in parallel, then the
objects are linked into ``attention_fa2_tiles_amd/libfa2tiles.so``.  Device
code is compiled for gfx950 only, with packed-fp32 instruction selection
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa2tiles.so")
SOURCES = ["attn_fwd.hip", "attn_fwd_fp8.hip", "attn_bwd.hip", "attn_f32.hip", "merge.hip", "lse_merge.hip", "api.cpp"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results in VGPRs: keeps loop-carried accumulators from being
        # copied between AGPRs and VGPRs on every iteration
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        f"-I{os.path.join(os.path.dirname(PKG), 'include')}",
    ]


def _compile(src, verbose):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc()] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{err}")
    if err and verbose:
        print(err)
    return obj


def build(verbose=False, jobs=None):
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print("built", path)
