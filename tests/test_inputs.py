"""Pins for the seeded input generator's storage formats (CPU only).

The float8 e5m2 storage used for fa_fwd_fp8's inputs is pinned to values
that follow from the OCP 8-bit floating-point format (sign, 5 exponent bits
with bias 15, 2 mantissa bits, subnormals below 2^-14, largest normal
57344) and to round-to-nearest-even ties.
"""

import numpy as np

from attention_fa2_tiles_amd.inputs import F8E5M2, draw, e5m2_bits_from_f32, from_storage, to_storage


def test_e5m2_decode_known_patterns():
    cases = {0x3C: 1.0, 0x38: 0.5, 0x40: 2.0, 0x3D: 1.25, 0x3E: 1.5, 0x3F: 1.75, 0xBC: -1.0,
             0x7B: 57344.0, 0x04: 2.0 ** -14, 0x01: 2.0 ** -16, 0x03: 3 * 2.0 ** -16, 0x00: 0.0}
    got = from_storage(np.array(list(cases), dtype=np.uint8), F8E5M2)
    np.testing.assert_array_equal(got, np.array(list(cases.values())))


def test_e5m2_rounding_nearest_even():
    x = np.array([1.0, 1.1, 1.125, 1.375, 1.2, -0.3, 3e-5, 1e6 / 1e6], dtype=np.float32)
    b = e5m2_bits_from_f32(x)
    v = from_storage(b, F8E5M2)
    # ties go to the even mantissa: 1.125 -> 1.0, 1.375 -> 1.5
    np.testing.assert_array_equal(v[:5], [1.0, 1.0, 1.0, 1.5, 1.25])
    # every result is one of the two neighbouring e5m2 values, the nearer one
    grid = from_storage(np.arange(256, dtype=np.uint8), F8E5M2)
    grid = grid[np.isfinite(grid)]
    for xi, vi in zip(x.astype(np.float64), v):
        assert np.abs(grid - xi).min() == abs(vi - xi)


def test_storage_round_trip_and_draw():
    t = draw(3, [("q", (2, 3, 16, 64), 1.0, F8E5M2)])["q"]
    assert t.storage.dtype == np.uint8
    np.testing.assert_array_equal(from_storage(t.storage, F8E5M2), t.f64)
    s2, f2 = to_storage(t.f64.astype(np.float32), F8E5M2)
    np.testing.assert_array_equal(s2, t.storage)  # stored values are fixed points of the rounding
