"""Thin ctypes binding of libfa2tiles.so (the C ABI in include/fa.h).

Every function here has the name and argument order of the C entry point and
only marshals arguments: a pointer argument may be a tensor-like object with
``data_ptr()`` (e.g. a torch CUDA tensor), a plain integer address, or None
(NULL).  ``stream`` may be None (torch's current stream when torch has
initialised CUDA, else the default stream), an integer hipStream_t, or an
object with a ``cuda_stream`` attribute.  A non-zero status raises FAError.

There is no fallback: if the library has not been built, ``load()`` raises.
"""

import ctypes
import os
import sys

F32, F16, BF16 = 0, 1, 2

STATUS = {
    0: "FA_OK",
    -1: "FA_ERR_NULL",
    -2: "FA_ERR_SHAPE",
    -3: "FA_ERR_DTYPE",
    -4: "FA_ERR_ALIGN",
    -5: "FA_ERR_WORKSPACE",
    -6: "FA_ERR_UNSUPPORTED",
    -7: "FA_ERR_HIP",
}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa2tiles.so")

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t

_SIGNATURES = {
    "fa_strerror": ([_I], ctypes.c_char_p),
    "fa_version": ([], _I),
    "fa_fwd": ([_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P], _I),
    "fa_fwd_fp8": ([_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P], _I),
    "fa_bwd_workspace_size": ([_I, _I, _I, _I, _I, _I], _Z),
    "fa_bwd": ([_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _I, _F, _P], _I),
    "fa_bwd_noalloc": ([_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P], _I),
    "fa_bwd_dlse": ([_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _I, _F, _P], _I),
    "fa_bwd_delta": ([_I, _P, _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "fa_bwd_dkdv": ([_I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P], _I),
    "fa_bwd_dq": ([_I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P], _I),
    "fa_bwd_dq_delta": ([_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P], _I),
    "fa_fwd_jvp": ([_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P], _I),
    "fa_fwd_jvp_tlse": ([_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P], _I),
    "pw_fwd": ([_I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P], _I),
    "pw_bwd_workspace_size": ([_I, _I, _I, _I, _I, _I], _Z),
    "pw_bwd": ([_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z,
                _I, _I, _I, _I, _I, _I, _F, _I, _P], _I),
    "pw_bwd_dlse": ([_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z,
                     _I, _I, _I, _I, _I, _I, _F, _I, _P], _I),
    "resmerge_fwd": ([_I, _P, _P, _P, _P, _P, _P, _I, _I, _F, _P], _I),
    "resmerge_bwd_workspace_size": ([_I, _I], _Z),
    "resmerge_bwd": ([_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _F, _P], _I),
    "resmerge_bwd_acc": ([_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _F, _I, _P], _I),
    "lse_merge_fwd": ([_I, _P, _P, _P, _P, _I, _I, _I, _P], _I),
    "lse_merge_bwd": ([_I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P], _I),
}

EXPORTS = tuple(_SIGNATURES)


class FAError(RuntimeError):
    def __init__(self, func, status, message):
        super().__init__(f"{func} failed: {message} ({status})")
        self.func = func
        self.status = status


def load(path=None):
    """Load the HIP library (once) and declare its signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FAError("load", -7, f"{p} is missing; build it with python -m attention_fa2_tiles_amd.build")
    lib = ctypes.CDLL(p)
    for name, (args, res) in _SIGNATURES.items():
        if path is not None and not hasattr(lib, name):
            continue  # an explicitly named (e.g. older) build may lack newer entry points
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        torch = sys.modules.get("torch")
        if torch is not None and torch.cuda.is_initialized():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(func, status):
    if status != 0:
        msg = load().fa_strerror(status).decode()
        raise FAError(func, status, msg)


def fa_strerror(status):
    return load().fa_strerror(status).decode()


def fa_version():
    return load().fa_version()


def fa_fwd(dtype, q, k, v, o, lse, B, H, M, N, D, causal, sm_scale, stream=None):
    _check("fa_fwd", load().fa_fwd(dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                   B, H, M, N, D, int(causal), sm_scale, _stream(stream)))


def fa_fwd_fp8(out_dtype, q, k, vt, o, lse, B, H, M, N, D, causal, sm_scale, stream=None):
    _check("fa_fwd_fp8", load().fa_fwd_fp8(out_dtype, _ptr(q), _ptr(k), _ptr(vt), _ptr(o), _ptr(lse),
                                           B, H, M, N, D, int(causal), sm_scale, _stream(stream)))


def fa_bwd_workspace_size(B, H, M, N, D, dtype):
    return load().fa_bwd_workspace_size(B, H, M, N, D, dtype)


def fa_bwd(dtype, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes,
           B, H, M, N, D, causal, sm_scale, stream=None):
    _check("fa_bwd", load().fa_bwd(dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace_bytes,
                                   B, H, M, N, D, int(causal), sm_scale, _stream(stream)))


def fa_bwd_noalloc(dtype, q, k, v, o, dout, lse, dq, dk, dv, B, H, M, N, D, causal, sm_scale, stream=None):
    _check("fa_bwd_noalloc", load().fa_bwd_noalloc(dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                                   _ptr(dq), _ptr(dk), _ptr(dv), B, H, M, N, D, int(causal),
                                                   sm_scale, _stream(stream)))


def fa_bwd_dlse(dtype, q, k, v, o, dout, lse, dlse, dq, dk, dv, workspace, workspace_bytes,
                B, H, M, N, D, causal, sm_scale, stream=None):
    _check("fa_bwd_dlse", load().fa_bwd_dlse(dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                             _ptr(dlse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                             workspace_bytes, B, H, M, N, D, int(causal), sm_scale,
                                             _stream(stream)))


def fa_bwd_delta(dtype, o, dout, dlse, delta, B, H, M, D, stream=None):
    _check("fa_bwd_delta", load().fa_bwd_delta(dtype, _ptr(o), _ptr(dout), _ptr(dlse), _ptr(delta), B, H, M, D,
                                               _stream(stream)))


def fa_bwd_dkdv(dtype, q, k, v, dout, lse, delta, dk, dv, B, H, M, N, D, causal, sm_scale, stream=None):
    _check("fa_bwd_dkdv", load().fa_bwd_dkdv(dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                                             _ptr(delta), _ptr(dk), _ptr(dv), B, H, M, N, D, int(causal),
                                             sm_scale, _stream(stream)))


def fa_bwd_dq(dtype, q, k, v, dout, lse, delta, dq, B, H, M, N, D, causal, sm_scale, stream=None):
    _check("fa_bwd_dq", load().fa_bwd_dq(dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                                         _ptr(delta), _ptr(dq), B, H, M, N, D, int(causal), sm_scale,
                                         _stream(stream)))


def fa_bwd_dq_delta(dtype, q, k, v, o, dout, lse, dlse, delta, dq, B, H, M, N, D, causal, sm_scale, stream=None):
    _check("fa_bwd_dq_delta", load().fa_bwd_dq_delta(dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                                     _ptr(lse), _ptr(dlse), _ptr(delta), _ptr(dq), B, H, M, N, D,
                                                     int(causal), sm_scale, _stream(stream)))


def fa_fwd_jvp(dtype, q, k, v, tq, tk, tv, o, lse, to, B, H, M, N, D, causal, sm_scale, stream=None):
    _check("fa_fwd_jvp", load().fa_fwd_jvp(dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk), _ptr(tv),
                                           _ptr(o), _ptr(lse), _ptr(to), B, H, M, N, D, int(causal),
                                           sm_scale, _stream(stream)))


def fa_fwd_jvp_tlse(dtype, q, k, v, tq, tk, tv, o, lse, to, tlse, B, H, M, N, D, causal, sm_scale, stream=None):
    _check("fa_fwd_jvp_tlse", load().fa_fwd_jvp_tlse(dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk),
                                                     _ptr(tv), _ptr(o), _ptr(lse), _ptr(to), _ptr(tlse),
                                                     B, H, M, N, D, int(causal), sm_scale, _stream(stream)))


def pw_fwd(dtype, q1, k1, q2, k2, v, o, lse, B, H, M, N, D, causal, sm_scale, w, stream=None):
    _check("pw_fwd", load().pw_fwd(dtype, _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(v), _ptr(o), _ptr(lse),
                                   B, H, M, N, D, int(causal), sm_scale, w, _stream(stream)))


def pw_bwd_workspace_size(B, H, M, N, D, dtype):
    return load().pw_bwd_workspace_size(B, H, M, N, D, dtype)


def pw_bwd(dtype, q1, k1, q2, k2, v, o, dout, lse, dq1, dk1, dq2, dk2, dv, workspace, workspace_bytes,
           B, H, M, N, D, causal, sm_scale, w, stream=None):
    _check("pw_bwd", load().pw_bwd(dtype, _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(v), _ptr(o), _ptr(dout),
                                   _ptr(lse), _ptr(dq1), _ptr(dk1), _ptr(dq2), _ptr(dk2), _ptr(dv),
                                   _ptr(workspace), workspace_bytes, B, H, M, N, D, int(causal), sm_scale, w,
                                   _stream(stream)))


def pw_bwd_dlse(dtype, q1, k1, q2, k2, v, o, dout, lse, dlse, dq1, dk1, dq2, dk2, dv, workspace, workspace_bytes,
                B, H, M, N, D, causal, sm_scale, w, stream=None):
    _check("pw_bwd_dlse", load().pw_bwd_dlse(dtype, _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(v), _ptr(o),
                                             _ptr(dout), _ptr(lse), _ptr(dlse), _ptr(dq1), _ptr(dk1), _ptr(dq2),
                                             _ptr(dk2), _ptr(dv), _ptr(workspace), workspace_bytes, B, H, M, N, D,
                                             int(causal), sm_scale, w, _stream(stream)))


def resmerge_fwd(dtype, x, q, y0, l0, y, lse, rows, D, eps, stream=None):
    _check("resmerge_fwd", load().resmerge_fwd(dtype, _ptr(x), _ptr(q), _ptr(y0), _ptr(l0), _ptr(y), _ptr(lse),
                                               rows, D, eps, _stream(stream)))


def resmerge_bwd_workspace_size(rows, D):
    return load().resmerge_bwd_workspace_size(rows, D)


def resmerge_bwd(dtype, x, q, y0, l0, gy, gl, gx, gq, gy0, gl0, workspace, workspace_bytes, rows, D, eps,
                 stream=None):
    _check("resmerge_bwd", load().resmerge_bwd(dtype, _ptr(x), _ptr(q), _ptr(y0), _ptr(l0), _ptr(gy), _ptr(gl),
                                               _ptr(gx), _ptr(gq), _ptr(gy0), _ptr(gl0), _ptr(workspace),
                                               workspace_bytes, rows, D, eps, _stream(stream)))


def resmerge_bwd_acc(dtype, x, q, y0, l0, gy, gl, gx, gq, gy0, gl0, workspace, workspace_bytes, rows, D, eps,
                     accumulate, stream=None):
    _check("resmerge_bwd_acc", load().resmerge_bwd_acc(dtype, _ptr(x), _ptr(q), _ptr(y0), _ptr(l0), _ptr(gy),
                                                       _ptr(gl), _ptr(gx), _ptr(gq), _ptr(gy0), _ptr(gl0),
                                                       _ptr(workspace), workspace_bytes, rows, D, eps,
                                                       int(accumulate), _stream(stream)))


def lse_merge_fwd(dtype, ys, lses, y, lse, S, rows, D, stream=None):
    _check("lse_merge_fwd", load().lse_merge_fwd(dtype, _ptr(ys), _ptr(lses), _ptr(y), _ptr(lse), S, rows, D,
                                                 _stream(stream)))


def lse_merge_bwd(dtype, ys, lses, gy, gl, gys, glses, S, rows, D, stream=None):
    _check("lse_merge_bwd", load().lse_merge_bwd(dtype, _ptr(ys), _ptr(lses), _ptr(gy), _ptr(gl), _ptr(gys),
                                                 _ptr(glses), S, rows, D, _stream(stream)))
