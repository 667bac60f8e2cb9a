"""GPU parity of the sparse GEMV over int8 rows with a per-row scale (run on an MI355X)."""
import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as asg
from activation_sparse_gemv_amd import _lib as L
from activation_sparse_gemv_amd import datagen
from oracle import quant, teal
from helpers import f64, rel_err, announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _int8(K, N, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(-127, 128, (K, N), generator=g, dtype=torch.int8)


@pytest.mark.parametrize("K,N", [(4096, 14336), (14336, 4096), (520, 1024), (4096, 64), (64, 8)])
def test_int8_rows_integer_valued_bit_exact(K, N):
    """Integer-valued x, int8 rows, power-of-two scales: every product and partial sum
    is an exact fp32 value, so Y equals the oracle bit for bit (split-K included)."""
    announce(f"int8 exact K={K} N={N}")
    x = datagen.int_valued((K,), 300 + K, -3, 3)
    q = _int8(K, N, K + N)
    sc = torch.from_numpy(np.exp2(np.random.default_rng(K).integers(-3, 1, K)).astype(np.float32))
    t = 1.5
    y = asg.as_threshold_gemv_i8(x.to(DEV), q.to(DEV), sc.to(DEV), t)
    ref = quant.masked_gemv_rows_int8(f64(x), q.numpy(), f64(sc), t)
    assert np.array_equal(f64(y), ref)


@pytest.mark.parametrize("K,N,xdt", [(4096, 14336, "bf16"), (14336, 4096, "f16"), (2056, 4096, "f32")])
def test_int8_rows_real_valued(K, N, xdt):
    """Student-t inputs, t at the median |x|, scales of quantized bf16 rows."""
    announce(f"int8 real K={K} N={N} {xdt}")
    x = datagen.student_t((K,), 400 + K, dtype=xdt)
    W = datagen.normal((K, N), 500 + K)
    q, s = quant.quantize_rows_int8(f64(W))
    qt, st = torch.from_numpy(q), torch.from_numpy(s.astype(np.float32))
    t = float(np.float32(np.median(np.abs(f64(x)))))
    y = asg.as_threshold_gemv_i8(x.to(DEV), qt.to(DEV), st.to(DEV), t)
    ref = quant.masked_gemv_rows_int8(f64(x), q, f64(st), t)
    assert rel_err(y, ref) < 2e-5
    # the dense flag reads every row
    yd = asg.as_threshold_gemv_i8(x.to(DEV), qt.to(DEV), st.to(DEV), t, flags=L.AS_FLAG_FORCE_DENSE)
    assert rel_err(yd, quant.masked_gemv_rows_int8(f64(x), q, f64(st), float("-inf"))) < 2e-5
    # deterministic
    assert torch.equal(y, asg.as_threshold_gemv_i8(x.to(DEV), qt.to(DEV), st.to(DEV), t))


def test_int8_rows_reject_unaligned_input():
    x = torch.zeros(4097, dtype=torch.bfloat16, device=DEV)[1:]
    q = torch.zeros((4096, 64), dtype=torch.int8, device=DEV)
    s = torch.ones(4096, dtype=torch.float32, device=DEV)
    with pytest.raises(L.ASError):
        asg.as_threshold_gemv_i8(x, q, s, 0.1)
