"""Seeded synthetic inputs for the activation-sparse decode path.

This module only draws numbers: weights, activations, priors and caches with
the shapes and value distributions of the five workloads.  It contains none of
the method's arithmetic (no thresholds, masks, ranks or products), so both the
GPU path and the CPU oracle can consume exactly the same bits from it.

Generation rules
----------------
* RNG: ``numpy.random.Generator(PCG64(seed))``; draws are cast to bf16/fp16
  through torch CPU tensors (round-to-nearest-even) and the cast bits are what
  every consumer sees.  Normal draws of more than 2^22 values take chunk k of
  2^22 values from the seed's stream advanced by k jumps (generated on threads;
  the values do not depend on the thread count).
* Seeds: ``seed = 10000*cfg + 100*layer + tag`` with the tags below.
* Weights: N(0, 0.02^2) drawn directly in the layout the kernels read.
* Activations: heavy-tailed (Laplace(0,1) or Student-t with 3 degrees of
  freedom), standing in for the heavy-tailed projection inputs that the TEAL
  slides (activation-distribution slide) report on C4 and that the
  intra-expert MoE summary (method section) reports inside experts.  No public
  corpus is used.
"""
from __future__ import annotations

import concurrent.futures as cf
import math
import os
from dataclasses import dataclass, field

import numpy as np
import torch

TAG = dict(w_gate=1, w_up=2, w_down=3, w_q=4, w_k=5, w_v=6, w_o=7, calib=8,
           decode=9, kv=10, prior=11, prompt=12, router=13, experts=14,
           shared=15, misc=16)

_TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def seed_for(cfg: int, layer: int, tag: str | int) -> int:
    t = TAG[tag] if isinstance(tag, str) else int(tag)
    return 10000 * int(cfg) + 100 * int(layer) + t


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(_TORCH_DT[dtype]).contiguous()


# Large draws are split into chunks of _CHUNK values; chunk k comes from the PCG64
# stream of the seed advanced by k jumps (PCG64.jumped(k)), so the values do not
# depend on how many threads generate them (chunk 0 is the plain stream).
_CHUNK = 1 << 22


def _workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def normal(shape, seed: int, std: float = 0.02, dtype: str = "bf16") -> torch.Tensor:
    """N(0, std^2) in the requested storage dtype (float32 draws, RNE cast)."""
    n = int(np.prod(shape))
    a = np.empty(n, dtype=np.float32)
    nch = max(1, (n + _CHUNK - 1) // _CHUNK)
    base = np.random.PCG64(seed)
    # every chunk's stream is set up before any draw (jumped() copies the state)
    gens = [np.random.Generator(base.jumped(k) if k else np.random.PCG64(seed)) for k in range(nch)]

    def fill(k: int) -> None:
        lo, hi = k * _CHUNK, min(n, (k + 1) * _CHUNK)
        gens[k].standard_normal(hi - lo, dtype=np.float32, out=a[lo:hi])

    if nch <= 1:
        fill(0)
    else:
        with cf.ThreadPoolExecutor(min(_workers(), nch)) as ex:
            list(ex.map(fill, range(nch)))
    a *= np.float32(std)
    return _cast(a.reshape(shape), dtype)


def laplace(shape, seed: int, scale: float = 1.0, dtype: str = "f16") -> torch.Tensor:
    a = _rng(seed).laplace(0.0, scale, size=shape)
    return _cast(a, dtype)


def student_t(shape, seed: int, nu: float = 3.0, dtype: str = "bf16") -> torch.Tensor:
    a = _rng(seed).standard_t(nu, size=shape)
    return _cast(a, dtype)


def uniform01(shape, seed: int) -> torch.Tensor:
    """Uniform[0,1) in fp32 (float32 draws)."""
    a = _rng(seed).random(size=shape, dtype=np.float32)
    return torch.from_numpy(a)


def int_valued(shape, seed: int, lo: int, hi: int, dtype: str = "bf16") -> torch.Tensor:
    """Integers drawn uniformly from [lo, hi], stored exactly in ``dtype``."""
    a = _rng(seed).integers(lo, hi + 1, size=shape).astype(np.float32)
    return _cast(a, dtype)


def with_specials(x: torch.Tensor, seed: int, frac: float = 0.01) -> torch.Tensor:
    """Copy of ``x`` with NaN, +-Inf, -0.0 and +0.0 planted at seeded positions."""
    y = x.clone().reshape(-1)
    n = y.numel()
    rng = _rng(seed)
    cnt = max(5, int(frac * n))
    pos = rng.choice(n, size=min(cnt, n), replace=False)
    vals = [float("nan"), float("inf"), float("-inf"), -0.0, 0.0]
    for j, p in enumerate(pos):
        y[int(p)] = vals[j % len(vals)]
    return y.reshape(x.shape)


# --------------------------------------------------------------------------
# Workload shapes
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class MLPShape:
    d_model: int
    d_ff: int
    w_dtype: str


CFG1 = MLPShape(512, 2048, "f16")        # small SwiGLU, fp16
CFG2 = MLPShape(4096, 14336, "bf16")     # Llama-3-8B-shaped MLP
CFG2_SWEEP = (0.0, 0.25, 0.40, 0.50, 0.65)
CFG3_ATTN = dict(d_model=4096, n_q=32, n_kv=8, head_dim=128, n_ctx=2048, n_blocks=32)
CFG4 = dict(d_model=4096, d_ff=14336, prompt=128, decode=256, keep=7168, lam=0.5)
CFG5 = dict(n_experts=128, d_model=2048, d_ff_e=768, top=8, keep=77, d_ff_shared=4096,
            tokens=(1, 4, 16))
N_CALIB = 256


def cfg3_sparsity(layer: int, n_blocks: int = 32) -> float:
    """Per-block sparsity schedule rising linearly from 30% to 60% with depth."""
    return 0.30 + 0.30 * layer / (n_blocks - 1)


# --------------------------------------------------------------------------
# Weight sets in kernel layout
# --------------------------------------------------------------------------
def mlp_weights_input_major(cfg: int, layer: int, shape: MLPShape):
    """Gate/up as ``[d_model, 2, d_ff]`` (row i = gate row i then up row i) and
    down as ``[d_ff, d_model]``: one input neuron's weights are one contiguous row."""
    d, f, dt = shape.d_model, shape.d_ff, shape.w_dtype
    wg = normal((d, f), seed_for(cfg, layer, "w_gate"), dtype=dt)
    wu = normal((d, f), seed_for(cfg, layer, "w_up"), dtype=dt)
    wgu = torch.stack([wg, wu], dim=1).contiguous()       # [d, 2, f]
    del wg, wu
    wd = normal((f, d), seed_for(cfg, layer, "w_down"), dtype=dt)
    return wgu, wd


def mlp_weights_neuron_major(cfg: int, layer: int, d_model: int, d_ff: int, dtype: str = "bf16"):
    """``[d_ff, 3, d_model]``: gate row, up row and down row of neuron j are adjacent.

    Gate and up are drawn as [d_ff, d_model] (neuron j's input weights); down is
    drawn as [d_ff, d_model] (neuron j's output weights)."""
    wg = normal((d_ff, d_model), seed_for(cfg, layer, "w_gate"), dtype=dtype)
    wu = normal((d_ff, d_model), seed_for(cfg, layer, "w_up"), dtype=dtype)
    wd = normal((d_ff, d_model), seed_for(cfg, layer, "w_down"), dtype=dtype)
    w = torch.stack([wg, wu, wd], dim=1).contiguous()     # [d_ff, 3, d_model]
    return w


def moe_weights(cfg: int = 5, layer: int = 0, n_experts: int = 128, d_model: int = 2048,
                d_ff_e: int = 768, d_ff_shared: int = 4096, dtype: str = "bf16"):
    """Router ``[d_model, E]``; routed experts gate/up ``[E, d_ff_e, 2, d_model]``
    (neuron-major) and down ``[E, d_ff_e, d_model]``; shared expert gate/up
    ``[d_model, 2, d_ff_shared]`` and down ``[d_ff_shared, d_model]`` (input-major)."""
    wr = normal((d_model, n_experts), seed_for(cfg, layer, "router"), dtype=dtype)
    s = seed_for(cfg, layer, "experts")
    wgu = normal((n_experts, d_ff_e, 2, d_model), s, dtype=dtype)
    wd = normal((n_experts, d_ff_e, d_model), s + 50, dtype=dtype)
    sg = normal((d_model, d_ff_shared), seed_for(cfg, layer, "shared"), dtype=dtype)
    su = normal((d_model, d_ff_shared), seed_for(cfg, layer, "shared") + 50, dtype=dtype)
    sgu = torch.stack([sg, su], dim=1).contiguous()
    sd = normal((d_ff_shared, d_model), seed_for(cfg, layer, "shared") + 70, dtype=dtype)
    return dict(w_router=wr, w_gate_up=wgu, w_down=wd, s_gate_up=sgu, s_down=sd)


def attn_weights(cfg: int, layer: int, d_model: int = 4096, n_q: int = 32, n_kv: int = 8,
                 head_dim: int = 128, dtype: str = "bf16"):
    """``w_qkv [d_model, (n_q + 2 n_kv) * head_dim]`` input-major (q | k | v columns)
    and ``w_o [n_q * head_dim, d_model]``."""
    q = normal((d_model, n_q * head_dim), seed_for(cfg, layer, "w_q"), dtype=dtype)
    k = normal((d_model, n_kv * head_dim), seed_for(cfg, layer, "w_k"), dtype=dtype)
    v = normal((d_model, n_kv * head_dim), seed_for(cfg, layer, "w_v"), dtype=dtype)
    wqkv = torch.cat([q, k, v], dim=1).contiguous()
    wo = normal((n_q * head_dim, d_model), seed_for(cfg, layer, "w_o"), dtype=dtype)
    return wqkv, wo


def kv_cache(cfg: int, layer: int, n_ctx: int = 2048, n_kv: int = 8, head_dim: int = 128):
    """K and V caches ``[n_ctx, n_kv, head_dim]`` bf16, N(0, 1)."""
    s = seed_for(cfg, layer, "kv")
    k = normal((n_ctx, n_kv, head_dim), s, std=1.0, dtype="bf16")
    v = normal((n_ctx, n_kv, head_dim), s + 50, std=1.0, dtype="bf16")
    return k, v
