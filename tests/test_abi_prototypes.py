"""The seven hot-path entry points of include/fa.h keep exactly the argument
lists of the boundary they implement (types, names and order), so a caller
written against that boundary passes every argument to the right slot; the
options beyond the pages live in separately named entry points with one
extra argument each.  Also checks that the ctypes binding declares the same
number of arguments as the header for every function.  CPU only."""

import os
import re

from attention_fa2_tiles_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

_ATTN = ["int B", "int H", "int M", "int N", "int D", "int causal", "float sm_scale"]

# (type, name) lists of the hot path's calls, in order.
EXPECTED = {
    "fa_fwd": ["int dtype", "const void* q", "const void* k", "const void* v", "void* o", "float* lse",
               *_ATTN, "void* stream"],
    "fa_bwd_workspace_size": ["int B", "int H", "int M", "int N", "int D", "int dtype"],
    "fa_bwd": ["int dtype", "const void* q", "const void* k", "const void* v", "const void* o",
               "const void* dout", "const float* lse", "void* dq", "void* dk", "void* dv",
               "void* workspace", "size_t workspace_bytes", *_ATTN, "void* stream"],
    "fa_fwd_jvp": ["int dtype", "const void* q", "const void* k", "const void* v", "const void* tq",
                   "const void* tk", "const void* tv", "void* o", "float* lse", "void* to", *_ATTN,
                   "void* stream"],
    "pw_fwd": ["int dtype", "const void* q1", "const void* k1", "const void* q2", "const void* k2",
               "const void* v", "void* o", "float* lse", *_ATTN, "int w", "void* stream"],
    "pw_bwd": ["int dtype", "const void* q1", "const void* k1", "const void* q2", "const void* k2",
               "const void* v", "const void* o", "const void* dout", "const float* lse", "void* dq1",
               "void* dk1", "void* dq2", "void* dk2", "void* dv", "void* workspace", "size_t workspace_bytes",
               *_ATTN, "int w", "void* stream"],
    "resmerge_fwd": ["int dtype", "const void* x", "const void* q", "const void* y0", "const float* l0",
                     "void* y", "float* lse", "int rows", "int D", "float eps", "void* stream"],
    "resmerge_bwd_workspace_size": ["int rows", "int D"],
    "resmerge_bwd": ["int dtype", "const void* x", "const void* q", "const void* y0", "const float* l0",
                     "const void* gy", "const float* gl", "void* gx", "float* gq", "void* gy0", "float* gl0",
                     "void* workspace", "size_t workspace_bytes", "int rows", "int D", "float eps",
                     "void* stream"],
}

# extended entry point -> (base, inserted argument, index it is inserted at)
EXTENDED = {
    "fa_bwd_dlse": ("fa_bwd", "const float* dlse", 7),
    "pw_bwd_dlse": ("pw_bwd", "const float* dlse", 9),
    "fa_fwd_jvp_tlse": ("fa_fwd_jvp", "float* tlse", 10),
    "resmerge_bwd_acc": ("resmerge_bwd", "int accumulate", 16),
}


def prototypes():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(?:int|size_t|const char\*)\s+(\w+)\s*\(([^)]*)\)\s*;", text):
        args = [" ".join(a.split()) for a in m.group(2).split(",")]
        args = [re.sub(r"\s*\*\s*", "* ", a).replace("* ", "* ", 1) for a in args if a and a != "void"]
        out[m.group(1)] = [re.sub(r"\*\s+", "* ", a) for a in args]
    return out


def test_hot_path_prototypes_exact():
    got = prototypes()
    for name, args in EXPECTED.items():
        assert name in got, name
        assert got[name] == args, f"{name}: header has {got[name]}"


def test_extended_entry_points_insert_one_argument():
    got = prototypes()
    for name, (base, extra, at) in EXTENDED.items():
        want = list(EXPECTED[base])
        want.insert(at, extra)
        assert got[name] == want, f"{name}: header has {got[name]}"


def test_binding_argument_counts_match_header():
    got = prototypes()
    for name, (argtypes, _) in lib._SIGNATURES.items():
        assert name in got, name
        assert len(argtypes) == len(got[name]), f"{name}: binding {len(argtypes)} vs header {len(got[name])}"
