"""Pins for the int8-row oracle (CPU only)."""
from fractions import Fraction

import numpy as np

from oracle import quant, teal


def test_int8_rows_exact_on_a_tiny_case_with_fractions():
    """K = 6, N = 3: the result equals the exact rational sum over the kept rows."""
    x = np.array([0.75, -2.0, 0.25, 3.5, -0.5, 1.0])
    q = np.array([[1, -2, 3], [127, 0, -127], [5, 5, 5], [-1, 2, -3], [100, -100, 7], [0, 1, 0]], dtype=np.int8)
    s = np.array([0.5, 0.125, 2.0, 0.25, 1.0, 4.0])
    t = 0.6
    y = quant.masked_gemv_rows_int8(x, q, s, t)
    want = [Fraction(0)] * 3
    for i in range(6):
        if abs(x[i]) > t:
            for j in range(3):
                want[j] += Fraction(x[i]) * Fraction(s[i]) * int(q[i, j])
    assert [Fraction(v) for v in y] == want


def test_int8_rows_equal_the_dequantized_masked_gemv():
    rng = np.random.default_rng(4)
    q = rng.integers(-127, 128, (300, 40)).astype(np.int8)
    s = rng.uniform(0.001, 0.05, 300)
    x = rng.standard_normal(300)
    t = float(np.median(np.abs(x)))
    y = quant.masked_gemv_rows_int8(x, q, s, t)
    np.testing.assert_allclose(y, teal.masked_gemv(x, q.astype(np.float64) * s[:, None], t), rtol=1e-12, atol=1e-12)


def test_the_mask_is_on_x_not_on_the_scaled_x():
    x = np.array([0.6, 0.4])
    q = np.array([[1], [1]], dtype=np.int8)
    s = np.array([0.1, 10.0])            # |x0 s0| = 0.06 < t < |x0|; |x1| < t < |x1 s1| = 4
    y = quant.masked_gemv_rows_int8(x, q, s, 0.5)
    assert y.tolist() == [0.6 * 0.1]


def test_row_quantizer_bounds():
    rng = np.random.default_rng(8)
    W = rng.standard_normal((50, 64)) * rng.uniform(0.01, 3, (50, 1))
    W[7] = 0.0
    q, s = quant.quantize_rows_int8(W)
    assert q.dtype == np.int8 and s[7] == 0 and not q[7].any()
    err = np.abs(W - q.astype(np.float64) * s[:, None])
    assert np.all(err <= s[:, None] / 2 + 1e-15)
    nz = s > 0
    assert np.all(np.abs(q[nz].astype(int)).max(axis=1) == 127)
