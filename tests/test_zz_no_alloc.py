"""The allocation-free MLP entry point (static per-device scratch) against the
entry point that takes a workspace: the same kernels on other memory, so the same
bits; two calls in a row, the second with a smaller input (other shapes: the
scratch is cleared for the new carve-up), then the first shape again."""
import pytest
import torch

import activation_sparse_gemv_amd as asg
from activation_sparse_gemv_amd import _lib as L
from activation_sparse_gemv_amd import datagen
from oracle import teal
from helpers import f64, announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(cfg, M):
    shape = datagen.CFG1 if cfg == 1 else datagen.CFG2
    wgu, wd = datagen.mlp_weights_input_major(cfg, 0, shape)
    w = asg.MLPWeights(wgu.to(DEV), wd.to(DEV))
    gen = datagen.laplace if cfg == 1 else datagen.student_t
    kw = dict(dtype="f16") if cfg == 1 else {}
    calib = gen((64, shape.d_model), datagen.seed_for(cfg, 0, "calib"), **kw)
    t_x, t_h, _ = teal.calibrate_mlp(f64(calib), f64(wgu[:, 0, :]), f64(wgu[:, 1, :]), 0.5, 0.5)
    x = gen((M, shape.d_model), datagen.seed_for(cfg, 7, "decode"), **kw).to(DEV)
    return w, x, float(t_x), float(t_h)


def test_noalloc_mlp_equals_workspace_entry_point():
    cases = [(2, 1), (1, 1), (2, 8), (2, 1)]     # the second call is smaller than the first
    for cfg, M in cases:
        announce(f"noalloc mlp cfg={cfg} M={M}")
        w, x, t_x, t_h = _case(cfg, M)
        for flags in (0, L.AS_FLAG_FORCE_DENSE):
            ref = asg.as_sparse_swiglu_mlp(x, w, t_x, t_h, flags=flags)
            Y = torch.full_like(ref, float("nan"))
            asg.api.as_sparse_swiglu_mlp_noalloc(x, w, Y, t_x, t_h, flags=flags)
            torch.cuda.synchronize()
            assert torch.equal(Y, ref), (cfg, M, flags)


def test_noalloc_rejects_oversized_calls():
    """A call whose workspace exceeds the static array is refused before any launch."""
    announce("noalloc oversized")
    shape = datagen.CFG2
    w = asg.MLPWeights(torch.empty((shape.d_model, 2, shape.d_ff), dtype=torch.bfloat16, device=DEV),
                       torch.empty((shape.d_ff, shape.d_model), dtype=torch.bfloat16, device=DEV))
    x = torch.zeros((16, shape.d_model), dtype=torch.bfloat16, device=DEV)
    Y = torch.empty((16, shape.d_model), dtype=torch.float32, device=DEV)
    with pytest.raises(L.ASError, match="scratch"):
        asg.api.as_sparse_swiglu_mlp_noalloc(x, w, Y, 1.0, 1.0)
