"""Pins for the magnitude-threshold oracle (CPU only)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import teal
from activation_sparse_gemv_amd import datagen


def _f64(t):
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------- worked example
def test_slide11_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "teal_slide11.json")))
    x = np.array(g["x"])
    m = teal.magnitude_mask(x, g["threshold"])
    assert m.astype(int).tolist() == g["mask"]
    assert teal.sparsify(x, g["threshold"]).tolist() == g["sparse_x"]
    # W = identity: y is sparse_x itself
    y = teal.masked_gemv(x, np.eye(5), g["threshold"])
    assert y.tolist() == g["sparse_x"]
    # the mask is unchanged by bf16 / fp16 rounding of x; kept values round as stated
    for dt, kept in (("bf16", [2.5, 1.796875]), ("f16", [2.5, 1.7998046875])):
        xb = _f64(datagen._cast(x, dt))
        mb = teal.magnitude_mask(xb, g["threshold"])
        assert mb.astype(int).tolist() == g["mask"]
        assert teal.sparsify(xb, g["threshold"])[[1, 3]].tolist() == kept


def test_threshold_is_strict():
    # slide 11 keeps |x| strictly above the threshold: a value equal to t is dropped
    x = np.array([0.5, -0.5, 0.5000001, -0.4999999])
    assert teal.magnitude_mask(x, 0.5).tolist() == [False, False, True, False]


def test_mask_specials():
    x = np.array([np.nan, np.inf, -np.inf, -0.0, 0.0, 1e-30])
    assert teal.magnitude_mask(x, 0.0).tolist() == [False, True, True, False, False, True]
    # t = -inf keeps every finite number, zeros included, and the infinities; NaN never
    assert teal.magnitude_mask(x, -np.inf).tolist() == [False, True, True, True, True, True]
    s = teal.sparsify(x, 0.0)
    assert np.isnan(s).sum() == 0 and s[0] == 0.0


# ---------------------------------------------------------------- masked GEMV
@pytest.mark.parametrize("M,K,N", [(1, 64, 64), (3, 200, 130), (5, 512, 1024)])
def test_gemv_minus_inf_is_matmul(M, K, N):
    x = _f64(datagen.student_t((M, K), 11, dtype="bf16"))
    W = _f64(datagen.normal((K, N), 12, dtype="bf16"))
    y = teal.masked_gemv(x, W, -np.inf)
    np.testing.assert_allclose(y, np.matmul(x, W), rtol=1e-13, atol=1e-15)
    # and column-by-column as a plain sum, to catch a transposed operand
    for n in (0, N // 2, N - 1):
        np.testing.assert_allclose(y[:, n], (x * W[:, n]).sum(axis=1), rtol=1e-12, atol=1e-15)


def test_gemv_all_masked_is_zero():
    x = _f64(datagen.student_t((2, 100), 3))
    W = _f64(datagen.normal((100, 40), 4))
    t = np.abs(x).max() + 1
    assert np.all(teal.masked_gemv(x, W, t) == 0.0)


def test_gemv_single_row():
    x = np.zeros(64)
    x[17] = 3.0
    x[5] = 0.25
    W = _f64(datagen.normal((64, 96), 5, dtype="bf16"))
    y = teal.masked_gemv(x, W, 0.5)
    assert np.array_equal(y, 3.0 * W[17])


def test_gemv_integer_exact():
    """Integer-valued inputs against exact Python-int arithmetic (no rounding anywhere)."""
    K, N = 300, 17
    x = _f64(datagen.int_valued((K,), 21, -8, 8))
    W = _f64(datagen.int_valued((K, N), 22, -4, 4))
    t = 3.0
    y = teal.masked_gemv(x, W, t)
    xi = [int(v) for v in x]
    Wi = [[int(v) for v in row] for row in W]
    for n in range(N):
        exact = sum(xi[i] * Wi[i][n] for i in range(K) if abs(xi[i]) > 3)
        assert y[n] == exact


# ---------------------------------------------------------------- calibration
@pytest.mark.parametrize("N", [10, 256, 1000, 4096])
@pytest.mark.parametrize("p", [0.25, 0.4, 0.5, 0.65, 0.3, 0.1])
def test_calibration_on_pool_1_to_N(N, p):
    pool = np.arange(1, N + 1, dtype=np.float64)
    rng = np.random.default_rng(N)
    pool = pool[rng.permutation(N)] * np.where(rng.random(N) < 0.5, -1, 1)
    t = teal.calibrate_threshold(pool, p)
    assert t == math.ceil(Fraction(str(p)) * N)      # closed form of the nearest rank
    kept = (np.abs(pool) > t).sum()
    dropped = N - kept
    assert dropped >= p * N - 1e-9 and dropped - 1 < p * N   # smallest count reaching p


def test_calibration_zero_and_specials():
    pool = np.array([3.0, -1.0, 2.0])
    assert teal.calibrate_threshold(pool, 0.0) == -np.inf
    assert teal.calibrate_threshold(pool, 1.0) == 3.0
    assert teal.calibrate_threshold(pool, 0.34) == 2.0   # ceil(1.02) = 2nd smallest |v|
    # ties in the pool: the realised sparsity may exceed p, never fall below it
    pool = np.array([1.0, 1.0, 1.0, 1.0, 2.0])
    t = teal.calibrate_threshold(pool, 0.5)
    assert t == 1.0 and (np.abs(pool) <= t).mean() >= 0.5


def test_calibration_rounds_to_fp32():
    pool = np.array([0.1, 0.2, 0.3])
    t = teal.calibrate_threshold(pool, 0.5)
    assert t.dtype == np.float32 and t == np.float32(0.2)


# ---------------------------------------------------------------- SwiGLU MLP
def test_silu_closed_forms():
    from scipy.special import expit
    z = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(teal.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    assert teal.silu(np.array([0.0]))[0] == 0.0
    assert teal.silu(np.array([800.0]))[0] == 800.0
    assert teal.silu(np.array([-800.0]))[0] == 0.0


def test_mlp_dense_special_case_matches_torch():
    d, f = 64, 192
    x = _f64(datagen.laplace((3, d), 31))
    Wg = _f64(datagen.normal((d, f), 32, dtype="f16"))
    Wu = _f64(datagen.normal((d, f), 33, dtype="f16"))
    Wd = _f64(datagen.normal((f, d), 34, dtype="f16"))
    r = teal.swiglu_mlp_threshold(x, Wg, Wu, Wd, -np.inf, -np.inf)
    xt = torch.from_numpy(x)
    ref = (torch.nn.functional.silu(xt @ torch.from_numpy(Wg)) * (xt @ torch.from_numpy(Wu))) @ torch.from_numpy(Wd)
    np.testing.assert_allclose(r["y"], ref.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(teal.dense_mlp(x, Wg, Wu, Wd), ref.numpy(), rtol=1e-12, atol=1e-15)


def test_mlp_masks_and_down_skip():
    d, f = 64, 128
    x = _f64(datagen.laplace((d,), 41))
    Wg = _f64(datagen.normal((d, f), 42))
    Wu = _f64(datagen.normal((d, f), 43))
    Wd = _f64(datagen.normal((f, d), 44))
    t_x = np.float32(0.7)
    r = teal.swiglu_mlp_threshold(x, Wg, Wu, Wd, t_x, 0.0)
    assert np.array_equal(r["m1"], np.abs(x) > 0.7)
    # dropping masked x entries == deleting those weight rows
    keep = np.flatnonzero(r["m1"])
    g2 = x[keep] @ Wg[keep]
    np.testing.assert_allclose(r["g"], g2, rtol=1e-12, atol=1e-16)
    # t_h picked between two |h| values: y == sum over kept neurons only
    a = np.sort(np.abs(r["h"]))
    t_h = np.float32((a[f // 2] + a[f // 2 + 1]) / 2)
    r = teal.swiglu_mlp_threshold(x, Wg, Wu, Wd, t_x, t_h)
    assert r["m2"].sum() == f - f // 2 - 1
    j = np.flatnonzero(r["m2"])
    np.testing.assert_allclose(r["y"], r["h"][j] @ Wd[j], rtol=1e-12, atol=1e-16)


def test_calibrate_mlp_sequential():
    d, f = 64, 128
    X = _f64(datagen.laplace((256, d), 51))
    Wg = _f64(datagen.normal((d, f), 52))
    Wu = _f64(datagen.normal((d, f), 53))
    t_x, t_h, h = teal.calibrate_mlp(X, Wg, Wu, 0.5, 0.5)
    assert (np.abs(X) <= t_x).mean() >= 0.5
    assert (np.abs(h) <= t_h).mean() >= 0.5
    # h pool was produced with t_x applied
    xs = np.where(np.abs(X) > t_x, X, 0)
    np.testing.assert_allclose(h, teal.silu(xs @ Wg) * (xs @ Wu), rtol=1e-12)


def test_bitmask_words():
    m = np.zeros(130, bool)
    m[[0, 63, 64, 129]] = True
    w = teal.bitmask_words(m)
    assert w.tolist() == [1 | (1 << 63), 1, 2]


def test_datagen_normal_is_chunk_and_thread_invariant():
    """Large normal draws are split into chunks of jumped PCG64 streams generated on
    threads: the values do not depend on the thread count, the first chunk is the
    plain stream of the seed, and an empty draw is empty."""
    import numpy as np
    import torch
    from activation_sparse_gemv_amd import datagen
    n = datagen._CHUNK + 1000
    a = datagen.normal((n,), 11, dtype="f32")
    b = datagen.normal((n,), 11, dtype="f32")
    assert torch.equal(a, b)
    first = np.random.Generator(np.random.PCG64(11)).standard_normal(1000, dtype=np.float32) * np.float32(0.02)
    assert np.array_equal(a[:1000].numpy(), first)
    tail = np.random.Generator(np.random.PCG64(11).jumped(1)).standard_normal(1000, dtype=np.float32) * np.float32(0.02)
    assert np.array_equal(a[datagen._CHUNK:].numpy(), tail)
    assert datagen.normal((0, 4), 3).numel() == 0
