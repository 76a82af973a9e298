"""Comparison rules between the HIP path and the fp64 oracle.

The bars (absolute max error for fp32; 1e-2 on O / LSE and 2e-2 relative to
max|ref| on gradients and tangents for fp16 / bf16) are the accuracy targets
this library is held to.  Two readings make them well defined:

* Outputs stored in fp16 / bf16 are compared with the oracle value rounded to
  that storage dtype, and an element passes if it is within max(tol, one
  ulp of the storage dtype at the reference).  A bf16 value of magnitude
  4..8 has a half-ulp of 0.0156, so even a correctly rounded result can sit
  more than 1e-2 from the unrounded reference; the one-ulp allowance covers
  exactly that and nothing more.
* "Relative to max|ref|" is max|gpu - ref| / max|ref| over the whole tensor.
* The fp32 bar of 1e-4 is absolute for tensors whose largest reference
  magnitude is at most 1 and scales with max|ref| beyond that: an fp32 value
  near 100 has an ulp of 7.6e-6, so a sum of a few thousand such terms cannot
  be held to 1e-4 absolute.  (The tiny fp32 attention workload has outputs of
  magnitude below a few units, where the two readings coincide up to that
  factor.)
"""

import numpy as np

from attention_fa2_tiles_amd.inputs import BF16, F16, F32, to_storage, from_storage

FP32_ATOL = 1e-4
OUT_ATOL = 1e-2
GRAD_REL = 2e-2


def fp32_scale(ref):
    finite = np.abs(ref[np.isfinite(ref)]) if np.size(ref) else np.zeros(1)
    return max(1.0, float(finite.max()) if finite.size else 1.0)


def rounded(ref, dtype):
    """fp64 reference rounded to the storage dtype (via fp32, RNE)."""
    if dtype == F32:
        return ref.astype(np.float32).astype(np.float64)
    s, _ = to_storage(np.asarray(ref, dtype=np.float32), dtype)
    return from_storage(s, dtype)


def ulp(v, dtype):
    mant = {F16: 10, BF16: 7, F32: 23}[dtype]
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    if dtype == F16:
        e = np.maximum(e, -14)
    return np.where(a > 0, 2.0 ** (e - mant), 2.0 ** (-14 - mant) if dtype == F16 else 0.0)


def check_output(name, got, ref, dtype, atol=None):
    """O-like tensors stored in the input dtype."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if dtype == F32:
        err = np.abs(got - ref).max() if got.size else 0.0
        bar = (atol or FP32_ATOL) * fp32_scale(ref)
        assert err <= bar, f"{name}: max abs err {err:.3e} > {bar:.3e}"
        return err
    rr = rounded(ref, dtype)
    bound = np.maximum(atol or OUT_ATOL, ulp(rr, dtype))
    diff = np.abs(got - rr)
    bad = diff > bound
    assert not bad.any(), (f"{name}: {bad.sum()} of {bad.size} elements out of tolerance; "
                           f"max diff {diff.max():.3e}; raw max abs vs fp64 {np.abs(got - ref).max():.3e}")
    return np.abs(got - ref).max()


def check_lse(name, got, ref, dtype):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf), f"{name}: -inf pattern differs"
    tol = FP32_ATOL if dtype == F32 else OUT_ATOL
    if (~ninf).any():
        err = np.abs(got[~ninf] - ref[~ninf]).max()
        assert err <= tol, f"{name}: max abs err {err:.3e} > {tol}"
        return err
    return 0.0


def check_grad(name, got, ref, dtype, zero_scale=None):
    """Gradients and tangents.  A reference that is exactly zero everywhere
    (a cancellation, e.g. dK with a single key, where dP - Delta = 0) has no
    scale of its own: zero_scale (a callable) then gives the magnitude of the
    summands that cancel, and the bar is GRAD_REL times that; without it the
    result must be exactly zero."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref).max() if got.size else 0.0
    if dtype == F32:
        bar = FP32_ATOL * fp32_scale(ref)
        assert err <= bar, f"{name}: max abs err {err:.3e} > {bar:.3e}"
        return err
    scale = np.abs(ref).max() if ref.size else 0.0
    if scale == 0.0:
        if zero_scale is None:
            assert err == 0.0, f"{name}: expected exact zeros, max abs {err:.3e}"
            return 0.0
        zs = zero_scale()
        assert err <= GRAD_REL * zs, f"{name}: max abs err {err:.3e} > {GRAD_REL} x {zs:.3e} (cancelled summands)"
        return err / zs if zs else 0.0
    rel = err / scale
    assert rel <= GRAD_REL, f"{name}: max abs err {err:.3e} = {rel:.3e} x max|ref| > {GRAD_REL}"
    return rel


def check_fp32_abs(name, got, ref, atol=FP32_ATOL):
    """The literal fp32 bar: max |gpu - ref| <= 1e-4, no scaling."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{name}: non-finite pattern differs"
    err = np.abs(got[fin] - ref[fin]).max() if fin.any() else 0.0
    assert err <= atol, f"{name}: max abs err {err:.3e} > {atol}"
    return err
