"""GPU parity of the threshold GEMV, the dense baseline and threshold calibration
against the fp64 oracle (run on an MI355X)."""
import json
import os

import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as asg
from activation_sparse_gemv_amd import _lib as L
from activation_sparse_gemv_amd import datagen
from oracle import teal
from helpers import TOL, f64, rel_err, bits_to_bool, announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(t):
    return t.to(DEV)


def _run(x, W, t, **kw):
    """With mask exports the whole input is compacted once per workgroup and split
    evenly; without them each slice masks its own range.  Both must agree."""
    out = asg.as_threshold_gemv(_dev(x), _dev(W), t, **kw)
    if kw.get("mask_out") and not kw.get("flags") and "Y" not in kw:
        y_range = asg.as_threshold_gemv(_dev(x), _dev(W), t)
        assert rel_err(y_range, f64(out[0])) < 1e-5
    return out


def test_slide11_example_on_gpu(golden_dir):
    announce("gemv slide-11 example")
    g = json.load(open(os.path.join(golden_dir, "teal_slide11.json")))
    x = torch.tensor(g["x"], dtype=torch.float32)
    W = datagen.normal((5, 64), 7, dtype="bf16")
    y, m = _run(x, W, g["threshold"], mask_out=True)
    torch.cuda.synchronize()
    assert bits_to_bool(m["bits"], 5)[0].astype(int).tolist() == g["mask"]
    assert m["nnz"].cpu().tolist() == [2]
    assert m["idx"][0, :2].cpu().tolist() == [1, 3]
    ref = teal.masked_gemv(f64(x), f64(W), g["threshold"])
    assert rel_err(y, ref) < 1e-6


@pytest.mark.parametrize("K,N", [(4096, 4096), (777, 200), (14336, 4096), (4096, 28672)])
def test_integer_valued_bit_exact(K, N):
    announce(f"gemv integer K={K} N={N}")
    x = datagen.int_valued((K,), 1000 + K, -8, 8)
    W = datagen.int_valued((K, N), 2000 + N, -4, 4)
    y = _run(x, W, 3.0)
    ref = teal.masked_gemv(f64(x), f64(W), 3.0)
    assert np.array_equal(f64(y), ref)                 # exact: integer sums < 2^24
    y2 = asg.as_dense_gemv(_dev(x), _dev(W))
    assert np.array_equal(f64(y2), f64(x) @ f64(W))


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("wdt,xdt", [("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32")])
def test_gemv_parity_shapes(M, wdt, xdt):
    K, N = 1000, 1352            # several tiles, ragged rows and a ragged column tile
    announce(f"gemv M={M} w={wdt} x={xdt}")
    x = datagen.student_t((M, K), 300 + M, dtype=xdt)
    W = datagen.normal((K, N), 301, dtype=wdt)
    t = float(teal.calibrate_threshold(f64(x), 0.5))
    y, m = _run(x, W, t, mask_out=True)
    ref = teal.masked_gemv(f64(x), f64(W), t)
    assert rel_err(y, ref) < TOL * 1e-2
    mask = teal.magnitude_mask(f64(x), t)
    assert np.array_equal(bits_to_bool(m["bits"], K), mask)
    assert m["nnz"].cpu().numpy().tolist() == mask.sum(axis=1).tolist()
    if M == 1:
        nnz = int(mask.sum())
        assert m["idx"][0, :nnz].cpu().numpy().tolist() == np.flatnonzero(mask[0]).tolist()


@pytest.mark.parametrize("M", [9, 12, 16])
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_gemv_mfma_batches(M, xdt):
    """9..16 tokens run on the matrix cores (bf16 weights); fp32 inputs go through the
    hi/lo bf16 split."""
    K, N = 1000, 1352
    announce(f"gemv mfma M={M} x={xdt}")
    x = datagen.student_t((M, K), 900 + M, dtype=xdt)
    W = datagen.normal((K, N), 901)
    t = float(teal.calibrate_threshold(f64(x), 0.5))
    y, m = _run(x, W, t, mask_out=True)
    assert rel_err(y, teal.masked_gemv(f64(x), f64(W), t)) < TOL * 1e-2
    assert np.array_equal(bits_to_bool(m["bits"], K), teal.magnitude_mask(f64(x), t))
    yd = asg.as_dense_gemv(_dev(x), _dev(W))
    assert rel_err(yd, f64(x) @ f64(W)) < TOL * 1e-2
    # Llama down-projection shape, batched
    x2 = datagen.student_t((M, 14336), 902 + M, dtype=xdt)
    W2 = datagen.normal((14336, 4096), 903)
    t2 = float(teal.calibrate_threshold(f64(x2), 0.5))
    assert rel_err(_run(x2, W2, t2), teal.masked_gemv(f64(x2), f64(W2), t2)) < TOL * 1e-2


def test_gemv_mfma_integer_bit_exact():
    announce("gemv mfma integer")
    K, N = 4096, 4096
    x = datagen.int_valued((16, K), 77, -8, 8)
    W = datagen.int_valued((K, N), 78, -4, 4)
    assert np.array_equal(f64(_run(x, W, 3.0)), teal.masked_gemv(f64(x), f64(W), 3.0))


@pytest.mark.parametrize("s", datagen.CFG2_SWEEP)
def test_gemv_llama_shapes_sweep(s):
    """Llama-3-8B-shaped projections (down: 14336 -> 4096, o: 4096 -> 4096) at each sparsity."""
    for K, N, tag in ((14336, 4096, "down"), (4096, 4096, "o")):
        announce(f"gemv {tag} s={s}")
        calib = datagen.student_t((256, K), 400 + K, dtype="bf16")
        t = float(teal.calibrate_threshold(f64(calib), s))
        x = datagen.student_t((1, K), 401 + K, dtype="bf16")
        W = datagen.normal((K, N), 402 + K, dtype="bf16")
        y, m = _run(x, W, t, mask_out=True)
        ref = teal.masked_gemv(f64(x), f64(W), t)
        assert rel_err(y, ref) < TOL * 1e-2
        assert np.array_equal(bits_to_bool(m["bits"], K), teal.magnitude_mask(f64(x), t))


def test_gemv_specials_and_edges():
    announce("gemv specials")
    K, N = 512, 256
    x = datagen.with_specials(datagen.student_t((1, K), 501), 502)
    x = x.masked_fill(torch.isinf(x), 0.0)           # NaN, -0.0 and +0.0 remain
    W = datagen.normal((K, N), 503)
    y, m = _run(x, W, 0.7, mask_out=True)
    ref = teal.masked_gemv(f64(x), f64(W), 0.7)
    assert not np.isnan(f64(y)).any()
    assert rel_err(y, ref) < 1e-5
    assert np.array_equal(bits_to_bool(m["bits"], K), teal.magnitude_mask(f64(x), 0.7))
    # t = -inf keeps zeros (and drops NaN)
    y, m = _run(x, W, float("-inf"), mask_out=True)
    assert np.array_equal(bits_to_bool(m["bits"], K), teal.magnitude_mask(f64(x), -np.inf))
    # everything masked -> exactly zero; accumulate leaves Y unchanged
    y = _run(x, W, 1e30)
    assert torch.count_nonzero(y).item() == 0
    Y0 = torch.randn(1, N, device=DEV)
    Y1 = Y0.clone()
    asg.as_threshold_gemv(_dev(x), _dev(W), 1e30, flags=L.AS_FLAG_ACCUMULATE, Y=Y1)
    assert torch.equal(Y0, Y1)
    # accumulate adds the product
    asg.as_threshold_gemv(_dev(x), _dev(W), 0.7, flags=L.AS_FLAG_ACCUMULATE, Y=Y1)
    assert rel_err(Y1, f64(Y0) + ref) < 1e-5
    # K = 1 and a single kept row
    x1 = torch.tensor([[2.0]], dtype=torch.bfloat16)
    W1 = datagen.normal((1, 64), 504)
    y1 = _run(x1, W1, 0.5)
    assert np.array_equal(f64(y1), 2.0 * f64(W1))


@pytest.mark.parametrize("K", [1000, 4096, 14336, 20000])
def test_gemv_unaligned_and_long_inputs(K):
    """x starting 2 bytes past a 16-byte boundary, and K beyond the register-chunk
    prologue, take the element-wise compaction path."""
    announce(f"gemv unaligned K={K}")
    buf = datagen.student_t((K + 1,), 650 + K)
    W = datagen.normal((K, 512), 651)
    xd = buf.to(DEV)[1:]
    t = float(teal.calibrate_threshold(f64(buf[1:]), 0.5))
    y, m = asg.as_threshold_gemv(xd, W.to(DEV), t, mask_out=True)
    ref = teal.masked_gemv(f64(buf[1:]), f64(W), t)
    assert rel_err(y, ref) < TOL * 1e-2
    mask = teal.magnitude_mask(f64(buf[1:]), t)
    nnz = int(mask.sum())
    assert m["idx"][0, :nnz].cpu().numpy().tolist() == np.flatnonzero(mask).tolist()
    # same launch plan (no exports: range-masked slices), aligned vs unaligned input:
    # identical rows in identical order, so bitwise equal
    y_u = asg.as_threshold_gemv(xd, W.to(DEV), t)
    y2 = asg.as_threshold_gemv(buf[1:].clone().to(DEV), W.to(DEV), t)
    assert torch.equal(y_u, y2)
    assert rel_err(y2, f64(y)) < 1e-5


@pytest.mark.parametrize("M,K,N", [(1, 14336, 4096), (3, 4096, 6144), (16, 4096, 4096), (1, 777, 200)])
def test_gemv_atomic_splitk(M, K, N):
    """AS_FLAG_ATOMIC_SPLITK: the row slices add into fp32 Y with atomics.  Integer-valued
    inputs sum exactly in any order, so Y is bit-exact (a NaN-filled Y is overwritten, and
    with AS_FLAG_ACCUMULATE the sum lands on Y's contents); real-valued inputs agree with
    the deterministic combine and the oracle."""
    announce(f"gemv atomic split-K M={M} K={K} N={N}")
    x = datagen.int_valued((M, K), 1300 + M, -8, 8)
    W = _dev(datagen.int_valued((K, N), 1301, -4, 4))
    ref = teal.masked_gemv(f64(x), f64(W.cpu()), 3.0)
    Y = torch.full((M, N), float("nan"), device=DEV)
    asg.as_threshold_gemv(_dev(x), W, 3.0, flags=L.AS_FLAG_ATOMIC_SPLITK, Y=Y)
    assert np.array_equal(f64(Y), ref)
    Y0 = datagen.int_valued((M, N), 1302, -100, 100).float().to(DEV)
    Y1 = Y0.clone()
    asg.as_threshold_gemv(_dev(x), W, 3.0, flags=L.AS_FLAG_ATOMIC_SPLITK | L.AS_FLAG_ACCUMULATE, Y=Y1)
    assert np.array_equal(f64(Y1), f64(Y0) + ref)
    xr = datagen.student_t((M, K), 1303)
    Wr = datagen.normal((K, N), 1304)
    ya = asg.as_threshold_gemv(_dev(xr), _dev(Wr), 1.0, flags=L.AS_FLAG_ATOMIC_SPLITK)
    yd = asg.as_threshold_gemv(_dev(xr), _dev(Wr), 1.0)
    assert rel_err(ya, f64(yd)) < 1e-5
    assert rel_err(ya, teal.masked_gemv(f64(xr), f64(Wr), 1.0)) < TOL * 1e-2
    yda = asg.as_dense_gemv(_dev(xr), _dev(Wr), flags=L.AS_FLAG_ATOMIC_SPLITK)
    assert rel_err(yda, f64(xr) @ f64(Wr)) < TOL * 1e-2


def test_gemv_determinism_and_nt_flag():
    announce("gemv determinism")
    K, N = 14336, 4096
    x = datagen.student_t((1, K), 601)
    W = _dev(datagen.normal((K, N), 602))
    xd = _dev(x)
    y1 = asg.as_threshold_gemv(xd, W, 1.0)
    y2 = asg.as_threshold_gemv(xd, W, 1.0)
    y3 = asg.as_threshold_gemv(xd, W, 1.0, flags=L.AS_FLAG_NO_NT_LOADS)
    assert torch.equal(y1, y2) and torch.equal(y1, y3)


def test_gemv_bf16_output_normwise():
    announce("gemv bf16 output")
    K, N = 4096, 4096
    x = datagen.student_t((1, K), 701)
    W = datagen.normal((K, N), 702)
    y = _run(x, W, 1.0, y_dtype=torch.bfloat16)
    ref = teal.masked_gemv(f64(x), f64(W), 1.0)
    # a bf16 result carries 8 significant bits: round-to-nearest costs up to 2^-8 of |y_i|
    # on top of the fp32 accumulation error (far below 1e-5 of max|y|)
    err = np.abs(f64(y) - ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max())


def test_dense_gemv_and_force_dense():
    announce("dense gemv")
    K, N = 4096, 6144
    x = datagen.student_t((2, K), 801)
    W = _dev(datagen.normal((K, N), 802))
    ref = f64(x) @ f64(W)
    y = asg.as_dense_gemv(_dev(x), W)
    assert rel_err(y, ref) < TOL * 1e-2
    y2 = asg.as_threshold_gemv(_dev(x), W, 5.0, flags=L.AS_FLAG_FORCE_DENSE)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("p", [0.0, 0.25, 0.4, 0.5, 0.65, 1.0])
def test_calibration_bit_exact(p):
    announce(f"calibrate p={p}")
    pool = datagen.student_t((256, 4096), 900, dtype="bf16")
    t = asg.as_calibrate_threshold(_dev(pool), p)
    ref = teal.calibrate_threshold(f64(pool), p)
    got = t.cpu().numpy()[0]
    assert got == ref or (np.isinf(got) and np.isinf(ref))
    # fp32 pool with ties and a NaN
    pool = torch.tensor([3.0, -1.0, 2.0, 2.0, -2.0, float("nan"), 0.5], dtype=torch.float32)
    for q in (0.1, 0.3, 0.5, 0.7, 0.85):
        got = asg.as_calibrate_threshold(_dev(pool), q).cpu().numpy()[0]
        assert got == teal.calibrate_threshold(f64(pool), q)


@pytest.mark.parametrize("n,dtype,offset", [(1000, "f16", 0), (1003, "f32", 1), (4099, "bf16", 3),
                                            (256 * 14336, "bf16", 0), (20_000_000, "bf16", 0),
                                            (3_000_001, "f32", 0), (777_777, "f16", 5)])
def test_calibration_sizes_and_layouts(n, dtype, offset):
    """The grid-wide radix select over pools of many workgroups (and more than the
    grid covers in one sweep), vector tails and unaligned pools (element offsets, so
    the element-wise path), against the sorted-pool oracle."""
    announce(f"calibrate n={n} {dtype} offset={offset}")
    buf = datagen.student_t((n + offset,), 950 + n % 97, dtype=dtype)
    pool_dev = _dev(buf)[offset:]
    ref_pool = f64(buf[offset:])
    for p in (0.05, 0.5, 0.97):
        got = asg.as_calibrate_threshold(pool_dev, p).cpu().numpy()[0]
        assert got == teal.calibrate_threshold(ref_pool, p), (n, dtype, offset, p)
    # the first and the last order statistic
    assert asg.as_calibrate_threshold(pool_dev, rank=1).cpu().numpy()[0] == np.float32(np.abs(ref_pool).min())
    assert asg.as_calibrate_threshold(pool_dev, rank=n).cpu().numpy()[0] == np.float32(np.abs(ref_pool).max())
