"""Magnitude thresholding (TEAL) in fp64: calibration, mask, masked GEMV, SwiGLU MLP.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def nearest_rank(p: float, n: int) -> int:
    """1-based nearest rank ``ceil(p * n)`` with ``p`` taken as the exact decimal it prints as."""
    if p <= 0:
        return 0
    return int(math.ceil(Fraction(repr(float(p))) * n))


def calibrate_threshold(pool: np.ndarray, p: float) -> np.float32:
    """Threshold t_p for target sparsity ``p`` from calibration values.

    TEAL slides, method slide ("TEAL: Training-Free Activation Sparsity"): t_p
    is decided from calibration data for the target sparsity; the entries of
    the input whose magnitude is small are zeroed.  Reading taken: t is the
    nearest-rank p-quantile of the pooled magnitudes, so that a fraction of at
    least p of the pool satisfies |v| <= t; p = 0 gives t = -inf (keep all).
    The pooled value is rounded up to the nearest fp32 (a pool of bf16/fp16
    inputs or of fp32 intermediates is already exact in fp32, so this only
    matters for fp64 pools, where rounding up keeps |v| <= t for the value at
    the nearest rank).
    """
    a = np.sort(np.abs(np.asarray(pool, dtype=np.float64)).ravel())
    if p <= 0:
        return np.float32(-np.inf)
    r = nearest_rank(p, a.size)
    r = min(max(r, 1), a.size)
    t = np.float32(a[r - 1])
    if np.float64(t) < a[r - 1]:
        t = np.nextafter(t, np.float32(np.inf))
    return t


def magnitude_mask(v: np.ndarray, t) -> np.ndarray:
    """``m_i = |v_i| > t`` (strict), compared exactly in fp64.

    TEAL slides, slide 11 (Hardware-Aware Acceleration): with threshold 0.5 only
    the elements with |x[i]| above 0.5 are computed.  NaN compares false
    (dropped); -0.0 is dropped for t >= 0; +-inf is kept for finite t.
    """
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        return np.abs(v) > np.float64(np.float32(t))


def sparsify(v: np.ndarray, t) -> np.ndarray:
    """``v * m`` with the masked entries set to exactly 0 (NaN/inf masked entries too)."""
    v = np.asarray(v, dtype=np.float64)
    m = magnitude_mask(v, t)
    return np.where(m, v, 0.0)


def masked_gemv(x: np.ndarray, W: np.ndarray, t) -> np.ndarray:
    """``y = (x * [|x| > t]) @ W`` with W input-major ``[K, N]``.

    TEAL slides, slide 11: sparse_x = x * mask, y = sparse_x @ W; the fused
    kernel loads only the weight rows whose input survives, which changes the
    bytes read but not the product.  ``x`` may be ``[K]`` or ``[M, K]``.
    """
    xs = sparsify(x, t)
    return xs @ np.asarray(W, dtype=np.float64)


def silu(z: np.ndarray) -> np.ndarray:
    """``z / (1 + exp(-z))`` in fp64 (the SiLU gate of the SwiGLU MLP)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_mlp_threshold(x, Wg, Wu, Wd, t_x, t_h):
    """Threshold-mode SwiGLU MLP of one or more decode tokens.

    TEAL slides, method slide: every projection input is thresholded, including
    the down-projection input, whose distribution the activation-distribution
    slide shows to be heavy-tailed.  Steps: m1 = |x| > t_x; g = (x*m1) Wg and
    u = (x*m1) Wu; h = silu(g) * u; m2 = |h| > t_h; y = (h*m2) Wd.  Glossary
    page (why sparsity saves compute): a zero intermediate neuron skips the
    matching row of the second FFN matrix.

    Wg, Wu: ``[d_model, d_ff]``; Wd: ``[d_ff, d_model]`` (all input-major).
    Returns a dict with m1, g, u, h, m2, y (fp64; masks bool).
    """
    x = np.asarray(x, dtype=np.float64)
    m1 = magnitude_mask(x, t_x)
    xs = np.where(m1, x, 0.0)
    g = xs @ np.asarray(Wg, dtype=np.float64)
    u = xs @ np.asarray(Wu, dtype=np.float64)
    h = silu(g) * u
    m2 = magnitude_mask(h, t_h)
    y = np.where(m2, h, 0.0) @ np.asarray(Wd, dtype=np.float64)
    return dict(m1=m1, g=g, u=u, h=h, m2=m2, y=y)


def down_stage(h, Wd, t_h):
    """Second stage alone, fed a given intermediate h: ``(h*[|h|>t_h]) @ Wd``."""
    return masked_gemv(h, Wd, t_h)


def calibrate_mlp(calib_x, Wg, Wu, p_x, p_h):
    """Sequential calibration of one MLP: t_x from |x|, then t_h from |h| of the
    calibration vectors with t_x already applied (reading: upstream sparsity on,
    so the realised sparsity matches the target at both inputs)."""
    t_x = calibrate_threshold(calib_x, p_x)
    x = np.asarray(calib_x, dtype=np.float64)
    xs = sparsify(x, t_x)
    h = silu(xs @ np.asarray(Wg, dtype=np.float64)) * (xs @ np.asarray(Wu, dtype=np.float64))
    t_h = calibrate_threshold(h, p_h)
    return t_x, t_h, h


def dense_mlp(x, Wg, Wu, Wd):
    """Dense SwiGLU ``(silu(x Wg) * (x Wu)) Wd`` -- the speedup denominator's function."""
    x = np.asarray(x, dtype=np.float64)
    h = silu(x @ np.asarray(Wg, dtype=np.float64)) * (x @ np.asarray(Wu, dtype=np.float64))
    return h @ np.asarray(Wd, dtype=np.float64)


def bitmask_words(m: np.ndarray) -> np.ndarray:
    """Pack a bool mask ``[..., n]`` into uint64 words: bit ``i % 64`` of word ``i // 64``."""
    m = np.asarray(m, dtype=bool)
    n = m.shape[-1]
    nw = (n + 63) // 64
    pad = np.zeros(m.shape[:-1] + (nw * 64,), dtype=bool)
    pad[..., :n] = m
    bits = pad.reshape(m.shape[:-1] + (nw, 64)).astype(np.uint64)
    w = np.zeros(m.shape[:-1] + (nw,), dtype=np.uint64)
    for b in range(64):
        w |= bits[..., b] << np.uint64(b)
    return w
