"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module holds no arithmetic of the attention or merge methods: it only
draws i.i.d. normal numbers with numpy's PCG64 generator, rounds them to a
storage dtype with round-to-nearest-even, and hands out the stored values
both as the raw storage array (for the device) and as float64 (for the fp64
oracle), so both sides see bit-identical inputs.

The workloads mirror the shapes the pages benchmark and test: batch x heads x
sequence x head-dim attention tensors with N(0, 1) entries, and the merge's
rows x hidden tensors (x, y0 ~ N(0, 1); l0 ~ N(0, 1); pseudo-query ~ N(0, 1/D)).
"""

from dataclasses import dataclass, field

import numpy as np

F32, F16, BF16 = 0, 1, 2  # same numbering as the C ABI's dtype codes
F8E5M2 = 3                # storage only: OCP float8 e5m2 bytes (fa_fwd_fp8's q, k, vt)
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16", F8E5M2: "f8e5m2"}


def bf16_bits_from_f32(a):
    """Round float32 -> bfloat16 (RNE); returns the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def f32_from_bf16_bits(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def e5m2_bits_from_f32(a):
    """Round float32 -> float8 e5m2 (via float16, then round-to-nearest-even
    on the low 8 bits of the float16 pattern: e5m2 is float16 with a 2-bit
    mantissa); returns uint8 bit patterns.  Inputs here are far below the
    e5m2 maximum (57344)."""
    h = np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16).astype(np.uint32)
    lsb = (h >> 8) & 1
    return ((h + 0x7F + lsb) >> 8).astype(np.uint8)


def f16_from_e5m2_bits(bits):
    return (np.asarray(bits, dtype=np.uint8).astype(np.uint16) << 8).view(np.float16)


def to_storage(a32, dtype):
    """Round a float32 array to the storage dtype.

    Returns (storage, as_f64): ``storage`` is float32, float16, or uint16 bf16
    bit patterns; ``as_f64`` is the exactly upcast value of what is stored."""
    if dtype == F32:
        s = np.ascontiguousarray(a32, dtype=np.float32)
        return s, s.astype(np.float64)
    if dtype == F16:
        s = np.ascontiguousarray(a32.astype(np.float16))
        return s, s.astype(np.float64)
    if dtype == BF16:
        s = bf16_bits_from_f32(a32)
        return s, f32_from_bf16_bits(s).astype(np.float64)
    if dtype == F8E5M2:
        s = e5m2_bits_from_f32(a32)
        return s, f16_from_e5m2_bits(s).astype(np.float64)
    raise ValueError(f"unknown dtype code {dtype}")


def from_storage(s, dtype):
    """Storage array -> float64 (inverse of the rounding step's view)."""
    if dtype == BF16:
        return f32_from_bf16_bits(np.asarray(s, dtype=np.uint16)).astype(np.float64)
    if dtype == F8E5M2:
        return f16_from_e5m2_bits(s).astype(np.float64)
    return np.asarray(s).astype(np.float64)


@dataclass
class Tensor:
    name: str
    storage: np.ndarray
    f64: np.ndarray
    dtype: int


@dataclass
class Draw:
    """A named, ordered set of seeded tensors."""
    seed: int
    tensors: dict = field(default_factory=dict)

    def __getitem__(self, k):
        return self.tensors[k]


def draw(seed, specs):
    """Draw tensors in the given order.

    ``specs`` is a list of (name, shape, std, dtype).  All values come from one
    PCG64 stream seeded with ``seed``, as float32 N(0, std^2), then rounded to
    ``dtype``."""
    rng = np.random.default_rng(seed)
    out = Draw(seed)
    for name, shape, std, dtype in specs:
        a = rng.standard_normal(size=shape, dtype=np.float32)
        if std != 1.0:
            a = (a * np.float32(std)).astype(np.float32)
        s, f = to_storage(a, dtype)
        out.tensors[name] = Tensor(name, s, f, dtype)
    return out


# ---------------------------------------------------------------------------
# Workloads.  Attention shapes are (B, H, M, N, D); sm_scale 0 means 1/sqrt(D).
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class AttnWorkload:
    name: str
    dtype: int
    B: int
    H: int
    M: int
    N: int
    D: int
    causal: bool
    seed: int
    sm_scale: float = 0.0

    def scale(self):
        return self.sm_scale if self.sm_scale != 0.0 else 1.0 / np.sqrt(self.D)

    def fwd_flops(self):
        """Counted work of one forward: 4*B*H*M*N*D, halved when causal.

        This is the flop convention of the gist's ``bench_flash_attention``
        (two matmuls of 2*M*N*D flops each per head)."""
        f = 4.0 * self.B * self.H * self.M * self.N * self.D
        return f * 0.5 if self.causal else f

    def bwd_flops(self):
        """Backward counted as 2.5x the forward (same benchmark convention)."""
        return 2.5 * self.fwd_flops()


@dataclass(frozen=True)
class MergeWorkload:
    name: str
    dtype: int
    rows: int
    D: int
    eps: float
    seed: int

    def fwd_bytes(self):
        """Algorithmic HBM bytes of one merge forward: read x, y0 (rows x D),
        q (D), l0 (rows, fp32); write y (rows x D) and lse (rows, fp32)."""
        es = 4 if self.dtype == F32 else 2
        return es * (3 * self.rows * self.D + self.D) + 8 * self.rows

    def bwd_bytes(self):
        """Algorithmic HBM bytes of one merge backward: read x, y0, gy, q, l0,
        gl; write gx, gy0, gl0 and the D-vector gq (fp32)."""
        es = 4 if self.dtype == F32 else 2
        return es * (5 * self.rows * self.D + self.D) + 12 * self.rows + 4 * self.D


@dataclass(frozen=True)
class LseMergeWorkload:
    """S attention partials (o, lse) of rows = B*H*M query rows, head dim D."""
    name: str
    dtype: int
    S: int
    rows: int
    D: int
    seed: int

    def fwd_bytes(self):
        """Algorithmic HBM bytes of one N-way merge forward: read ys
        (S x rows x D) and lses (S x rows, fp32); write y (rows x D) and lse."""
        es = 4 if self.dtype == F32 else 2
        return es * (self.S + 1) * self.rows * self.D + 4 * (self.S + 1) * self.rows

    def bwd_bytes(self):
        """Algorithmic HBM bytes of one N-way merge backward: read ys, lses,
        gy, gl; write gys (S x rows x D) and glses (S x rows)."""
        es = 4 if self.dtype == F32 else 2
        return es * (2 * self.S + 1) * self.rows * self.D + 4 * (2 * self.S + 1) * self.rows


WORKLOADS = {
    "tiny_f32": AttnWorkload("tiny_f32", F32, 1, 2, 128, 128, 64, False, 1, 0.125),
    "causal_bf16_b4h16_s2048_d128": AttnWorkload(
        "causal_bf16_b4h16_s2048_d128", BF16, 4, 16, 2048, 2048, 128, True, 2),
    "noncausal_bf16_b1h32_s8192_d128": AttnWorkload(
        "noncausal_bf16_b1h32_s8192_d128", BF16, 1, 32, 8192, 8192, 128, False, 2),
    "jvp_f16_b4h16_s1024_d64_causal": AttnWorkload(
        "jvp_f16_b4h16_s1024_d64_causal", F16, 4, 16, 1024, 1024, 64, True, 3),
    "jvp_f16_b4h16_s1024_d64": AttnWorkload(
        "jvp_f16_b4h16_s1024_d64", F16, 4, 16, 1024, 1024, 64, False, 3),
    "piecewise_f16_b2h16_s4096_d64_w1024": AttnWorkload(
        "piecewise_f16_b2h16_s4096_d64_w1024", F16, 2, 16, 4096, 4096, 64, True, 4),
}
PIECEWISE_W = 1024

MERGE_WORKLOAD = MergeWorkload("merge_bf16_rows32768_d4096", BF16, 8 * 4096, 4096, 1e-6, 5)

# Split-KV combine of the causal headline shape (B4 H16 2048 query rows,
# D128) over 4 key splits.
LSE_MERGE_WORKLOAD = LseMergeWorkload("lse_merge_bf16_s4_rows131072_d128", BF16, 4, 4 * 16 * 2048, 128, 6)


def attn_inputs(wl, names=("q", "k", "v", "do"), seed=None):
    """Seeded attention tensors: q-like [B,H,M,D] and k-like [B,H,N,D]."""
    qshape = (wl.B, wl.H, wl.M, wl.D)
    kshape = (wl.B, wl.H, wl.N, wl.D)
    qlike = {"q", "do", "tq", "q1", "q2"}
    specs = [(n, qshape if n in qlike else kshape, 1.0, wl.dtype) for n in names]
    return draw(wl.seed if seed is None else seed, specs)


def lse_merge_inputs(wl, seed=None):
    """Seeded N-way merge tensors: ys, lses (N(0, 4): partials of different
    weight), gy, gl."""
    specs = [
        ("ys", (wl.S, wl.rows, wl.D), 1.0, wl.dtype),
        ("lses", (wl.S, wl.rows), 2.0, F32),
        ("gy", (wl.rows, wl.D), 1.0, wl.dtype),
        ("gl", (wl.rows,), 1.0, F32),
    ]
    return draw(wl.seed if seed is None else seed, specs)


def merge_inputs(wl, seed=None):
    """Seeded merge tensors in a fixed order: x, y0, l0, q, gy, gl."""
    r, D = wl.rows, wl.D
    specs = [
        ("x", (r, D), 1.0, wl.dtype),
        ("y0", (r, D), 1.0, wl.dtype),
        ("l0", (r,), 1.0, F32),
        ("q", (D,), 1.0 / np.sqrt(D), wl.dtype),
        ("gy", (r, D), 1.0, wl.dtype),
        ("gl", (r,), 1.0, F32),
    ]
    return draw(wl.seed if seed is None else seed, specs)
