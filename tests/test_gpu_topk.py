"""GPU parity of the exact top-k masks (value and GLASS rank-blend modes): the
index sets and bitmasks must equal the oracle's bit for bit."""
import json
import os

import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as asg
from activation_sparse_gemv_amd import datagen
from oracle import topk
from helpers import bits_to_bool, announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu_topk(score, k, prior=None, lam=0.5):
    s = torch.as_tensor(np.asarray(score, dtype=np.float32)).to(DEV)
    p = None if prior is None else torch.as_tensor(np.asarray(prior, dtype=np.float32)).to(DEV)
    mask, idx = asg.as_topk_mask(s, k, prior=p, lam=lam)
    return mask, idx


def _check_rows(scores, k, prior=None, lam=0.5):
    scores = np.atleast_2d(scores).astype(np.float32)
    rows, n = scores.shape
    pr = None if prior is None else np.atleast_2d(prior).astype(np.float32)
    mask, idx = _gpu_topk(scores, k, pr, lam)
    m = bits_to_bool(mask, n)
    for r in range(rows):
        if pr is None:
            ref = topk.value_topk(scores[r].astype(np.float64), k)
        else:
            ref = topk.glass_topk(scores[r].astype(np.float64), pr[r].astype(np.float64), lam, k)
        assert idx[r].cpu().numpy().tolist() == ref.tolist(), (r, n, k)
        assert np.array_equal(m[r], topk.mask_from_index(ref, n)), (r, n, k)


def test_hand_cases(golden_dir):
    announce("topk hand cases")
    g = json.load(open(os.path.join(golden_dir, "topk_cases.json")))
    for c in g["value_topk"]:
        s = np.array([float(v) for v in c["scores"]], dtype=np.float32)
        mask, idx = _gpu_topk(s, c["k"])
        assert idx.cpu().numpy().tolist() == c["idx"], c
    for c in g["blend"]:
        for k, ref in c["k"].items():
            mask, idx = _gpu_topk(np.array(c["local"]), int(k), np.array(c["prior"]), c["lambda"])
            assert idx.cpu().numpy().tolist() == ref, (c, k)


@pytest.mark.parametrize("n", [1, 5, 63, 64, 65, 1000, 1025, 4097])
def test_value_topk_ties_and_specials(n):
    announce(f"topk value n={n}")
    rng = np.random.default_rng(n)
    s = rng.integers(-4, 5, size=(3, n)).astype(np.float32)       # heavy ties
    if n >= 5:
        s[0, rng.choice(n, size=min(5, n), replace=False)] = [np.nan, -0.0, 0.0, np.inf, -np.inf][:min(5, n)]
    s[2] = rng.standard_normal(n).astype(np.float32)
    for k in sorted({0, 1, n // 3, n // 2, max(n - 1, 0), n}):
        _check_rows(s, k)


def test_value_topk_expert_shape():
    """keep 77 of 768 per (token, expert) row, 128 rows."""
    announce("topk expert shape")
    rng = np.random.default_rng(5)
    s = np.abs(rng.standard_t(3, size=(128, 768))).astype(np.float32)
    _check_rows(s, 77)


@pytest.mark.parametrize("lam", [0.5, 0.0, 1.0, 0.3])
def test_blend_glass_workload(lam):
    """n = 14336 FFN neurons, keep 7168: local = mean |h| style scores with ties, prior
    uniform fp32 with natural collisions."""
    announce(f"topk blend lam={lam}")
    n, k = 14336, 7168
    local = np.round(np.abs(np.random.default_rng(11).standard_t(3, n)), 3).astype(np.float32)
    prior = datagen.uniform01((n,), datagen.seed_for(4, 0, "prior")).numpy()
    _check_rows(local, k, prior, lam)
    for kk in (1, 100, n - 1, n):
        _check_rows(local, kk, prior, lam)


def test_blend_multi_row_and_ties():
    announce("topk blend rows")
    rng = np.random.default_rng(3)
    local = rng.integers(0, 5, size=(4, 300)).astype(np.float32)
    prior = rng.integers(0, 5, size=(4, 300)).astype(np.float32)
    for k in (0, 1, 150, 299, 300):
        _check_rows(local, k, prior, 0.5)


@pytest.mark.parametrize("n", [16384, 20000, 40000])
def test_blend_large_n(n):
    """Rank blend past the GLASS size, up to scores staged outside LDS (n > 32768),
    with ties, -0.0 / +0.0 and NaN, two rows, several k, called repeatedly (the rank
    counts are cleared by each call for the next)."""
    announce(f"topk blend n={n}")
    rng = np.random.default_rng(n)
    local = rng.integers(0, 50, size=(2, n)).astype(np.float32)
    prior = rng.random((2, n), dtype=np.float32)
    local[0, :7] = [np.nan, -0.0, 0.0, np.inf, -np.inf, np.nan, 0.0]
    prior[1, 3:6] = prior[1, 2]
    for k in (1, n // 2, n - 1):
        _check_rows(local, k, prior, 0.5)
    _check_rows(local, n // 3, prior, 0.25)
