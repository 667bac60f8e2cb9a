"""Decoder block with magnitude-thresholded projection inputs, in fp64.

Test infrastructure only (see the package docstring).

Readings taken (the pages describe no block in code): pre-norm RMSNorm with
unit gain and eps 1e-5; no rotary embedding; grouped-query attention where
query head h reads key/value head h // (n_q / n_kv); the keys are the cached
context plus the current token's own key; thresholds are one per distinct
projection input (q/k/v share one, then o, gate/up, down).
"""
from __future__ import annotations

import numpy as np

from .teal import sparsify, silu


def rmsnorm(x, eps: float = 1e-5):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def softmax(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def gqa_decode_attention(q, k_cache, v_cache, k_new, v_new):
    """One decode token: q ``[n_q, hd]``, caches ``[n_ctx, n_kv, hd]``, new k/v
    ``[n_kv, hd]``.  Dense softmax attention over n_ctx + 1 keys, scale
    1/sqrt(hd).  Returns o ``[n_q * hd]`` (heads concatenated)."""
    q = np.asarray(q, dtype=np.float64)
    n_q, hd = q.shape
    K = np.concatenate([np.asarray(k_cache, np.float64), np.asarray(k_new, np.float64)[None]], 0)
    V = np.concatenate([np.asarray(v_cache, np.float64), np.asarray(v_new, np.float64)[None]], 0)
    n_kv = K.shape[1]
    grp = n_q // n_kv
    o = np.zeros((n_q, hd))
    for h in range(n_q):
        kh = h // grp
        s = (K[:, kh, :] @ q[h]) / np.sqrt(hd)
        p = softmax(s)
        o[h] = p @ V[:, kh, :]
    return o.reshape(-1)


def decoder_block(x, wqkv, wo, wgu, wd, k_cache, v_cache, t, n_q=32, n_kv=8, hd=128):
    """Decode tokens through one block with thresholded projection inputs.

    TEAL slides, method slide: the inputs of the attention and MLP blocks' linear
    layers are magnitude-thresholded; the attention core stays dense.
    ``x`` is one token ``[d]`` or independent tokens ``[T, d]`` (each token is the
    same computation; the rows only share the matrix products).
    ``t`` = dict(qkv=, o=, gu=, d=) fp32 thresholds.  Weights input-major:
    wqkv [d, (n_q + 2 n_kv) hd], wo [n_q hd, d], wgu [d, 2, d_ff], wd [d_ff, d].
    Returns a dict of every intermediate and ``out`` (rows = tokens).
    """
    x = np.asarray(x, dtype=np.float64)
    xn = rmsnorm(x)
    xs = sparsify(xn, t["qkv"])
    qkv = xs @ np.asarray(wqkv, np.float64)

    def attend(row):
        q = row[: n_q * hd].reshape(n_q, hd)
        kn = row[n_q * hd: (n_q + n_kv) * hd].reshape(n_kv, hd)
        vn = row[(n_q + n_kv) * hd:].reshape(n_kv, hd)
        return gqa_decode_attention(q, k_cache, v_cache, kn, vn)

    o = attend(qkv) if qkv.ndim == 1 else np.stack([attend(r) for r in qkv])
    y_att = sparsify(o, t["o"]) @ np.asarray(wo, np.float64)
    h1 = x + y_att
    xn2 = rmsnorm(h1)
    xs2 = sparsify(xn2, t["gu"])
    W = np.asarray(wgu, np.float64)
    hmid = silu(xs2 @ W[:, 0, :]) * (xs2 @ W[:, 1, :])
    y_mlp = sparsify(hmid, t["d"]) @ np.asarray(wd, np.float64)
    out = h1 + y_mlp
    return dict(xn=xn, qkv=qkv, o=o, y_att=y_att, h1=h1, xn2=xn2, h=hmid, y_mlp=y_mlp, out=out)
