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
SOURCES = ["attn_fwd.hip", "attn_fwd_fp8.hip", "attn_bwd.hip", "attn_generic.hip", "merge.hip", "lse_merge.hip",
           "noalloc.hip", "api.cpp"]
# Sources compiled in several parts (each part instantiates a share of the
# kernels, selected by a macro), so the parts compile in parallel.
PARTS = {"attn_bwd.hip": ("FA_BWD_PART", 9), "attn_fwd.hip": ("FA_FWD_PART", 5)}
# MFMA results in VGPRs: keeps loop-carried accumulators from being copied
# between AGPRs and VGPRs on every iteration.  Every unit but the parts
# listed in AGPR_PARTS, whose kernels run one wave per SIMD with more
# accumulator registers than the 256 VGPRs (the D = 256 backward passes).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
AGPR_PARTS = {"attn_bwd.hip": {5, 6, 7, 8}}


def units():
    """(source, extra flags, object name) of every translation unit."""
    out = []
    for src in SOURCES:
        if src in PARTS:
            macro, n = PARTS[src]
            for i in range(n):
                form = [] if i in AGPR_PARTS.get(src, ()) else VGPR_FORM
                out.append((src, [f"-D{macro}={i}"] + form, f"{src}.part{i}.o"))
        else:
            out.append((src, list(VGPR_FORM), src + ".o"))
    return out
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
        f"-I{os.path.join(os.path.dirname(PKG), 'include')}",
    ]


def _compile(unit, verbose):
    src, extra, name = unit
    obj = os.path.join(BUILD, name)
    cmd = [hipcc()] + compile_flags() + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
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


def _stale(unit):
    """Whether a unit's object is older than its source or any header."""
    src, _, name = unit
    obj = os.path.join(BUILD, name)
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    deps += [os.path.join(os.path.dirname(PKG), "include", f)
             for f in os.listdir(os.path.join(os.path.dirname(PKG), "include"))]
    return max(os.path.getmtime(d) for d in deps) > os.path.getmtime(obj)


def build(verbose=False, jobs=None, incremental=False):
    """Compile every source and link the shared library; returns its path.
    incremental=True recompiles only units older than their sources (a
    development shortcut; the default always recompiles everything)."""
    os.makedirs(BUILD, exist_ok=True)
    us = units()
    todo = [u for u in us if _stale(u)] if incremental else us
    # longest units first
    todo.sort(key=lambda u: (u[0] not in PARTS, u[0] != "attn_bwd.hip"))
    jobs = jobs or min(max(1, len(todo)), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda u: _compile(u, verbose), todo))
    objs = [os.path.join(BUILD, name) for _, _, name in us]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized(out_dir=None, verbose=False):
    """A copy of the library whose host-side C ABI layer (api.cpp: argument
    validation and launch set-up) is compiled by g++ with AddressSanitizer
    and UndefinedBehaviorSanitizer; the kernel objects are the ordinary ones
    from _build/ (build() must have run).  For CPU tests of rejected calls
    only: load it in a process that preloads g++'s libasan.  Returns the
    library path."""
    out_dir = out_dir or BUILD
    os.makedirs(out_dir, exist_ok=True)
    objs = [os.path.join(BUILD, name) for src, _, name in units() if src != "api.cpp"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise FileNotFoundError(f"kernel objects missing (run build() first): {missing}")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]
    api_obj = os.path.join(out_dir, "api_hostsan.o")
    cmd = (["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
            f"-I{os.path.join(os.path.dirname(PKG), 'include')}"] + san
           + ["-c", os.path.join(CSRC, "api.cpp"), "-o", api_obj])
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized api.cpp failed:\n{r.stderr}")
    lib = os.path.join(out_dir, "libfa2tiles_hostsan.so")
    cmd = ["g++", "-shared", "-fPIC"] + san + ["-o", lib, api_obj] + objs + [f"-L{rocm}/lib", "-lamdhip64",
                                                                             f"-Wl,-rpath,{rocm}/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    return lib


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print("built", path)
