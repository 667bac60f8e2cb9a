"""Tensor-level binding of libactsparse: argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: it checks tensor placement, allocates outputs and the
workspace with torch (device memory is torch's), and passes raw pointers and
torch's current HIP stream to the library.  Workspaces are cached per
(entry point, shape) and device, zero-filled once; the library leaves their
counters at zero after every call, so reuse on one stream is safe.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from fractions import Fraction
from typing import Optional

import torch

from . import _lib as L

_DT = {torch.float16: L.AS_F16, torch.bfloat16: L.AS_BF16, torch.float32: L.AS_F32}
_WS: dict = {}


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libactsparse operates on device tensors only (no CPU path exists)")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def workspace(key, nbytes: int, device: torch.device) -> torch.Tensor:
    """Zero-filled workspace cached per call shape (the library's launch plan, and so
    the workspace's carve-up, is a function of the shapes alone)."""
    k = (key, nbytes, str(device))
    ws = _WS.get(k)
    if ws is None:
        ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)
        _WS[k] = ws
    return ws


def as_version() -> int:
    return L.load().as_version()


def as_calibrate_threshold(pool: torch.Tensor, p: float | None = None, rank: int | None = None) -> torch.Tensor:
    """Threshold for target sparsity p (the decimal p is passed to the library as the
    exact rational it prints as) or for an explicit 1-based rank (passed as the
    rational rank / n) from a calibration pool; returns a 1-element fp32 device tensor."""
    _need_cuda(pool)
    n = pool.numel()
    q = Fraction(int(rank), n) if rank is not None else Fraction(repr(float(p))) if p > 0 else Fraction(0)
    out = torch.empty(1, dtype=torch.float32, device=pool.device)
    lib = L.load()
    nb = lib.as_calibrate_threshold_ws_size(n)
    ws = workspace(("calibrate",), nb, pool.device)
    L.check(lib.as_calibrate_threshold(_ptr(pool), _dt(pool), n, q.numerator, q.denominator, _ptr(out), _ptr(ws), nb,
                                       _stream(pool.device)), "as_calibrate_threshold")
    return out


def _mask_bufs(M: int, n: int, device, want_idx: bool):
    nw = (n + 63) // 64
    bits = torch.zeros((M, nw), dtype=torch.int64, device=device)
    nnz = torch.zeros(M, dtype=torch.int32, device=device)
    idx = torch.full((M, n), -1, dtype=torch.int32, device=device) if want_idx else None
    return dict(bits=bits, nnz=nnz, idx=idx)


def _mask_struct(d) -> L.ASMaskOut:
    if d is None:
        return L.ASMaskOut(None, None, None)
    return L.ASMaskOut(_ptr(d.get("bits")), _ptr(d.get("idx")), _ptr(d.get("nnz")))


def as_threshold_gemv(X: torch.Tensor, W: torch.Tensor, t: float, y_dtype=torch.float32,
                      flags: int = 0, mask_out: bool = False, Y: torch.Tensor | None = None):
    """Y[m] = sum_{i: |X[m,i]| > t} X[m,i] W[i,:].  X [M,K] or [K]; W [K,N]."""
    squeeze = X.dim() == 1
    X2 = X.reshape(1, -1) if squeeze else X
    _need_cuda(X2, W, Y)
    M, K = X2.shape
    K2, N = W.shape
    if K2 != K:
        raise ValueError(f"X has K={K} but W has {K2} rows")
    if Y is None:
        Y = torch.empty((M, N), dtype=y_dtype, device=X.device)
    lib = L.load()
    nb = lib.as_threshold_gemv_ws_size(M, K, N)
    ws = workspace(("gemv", M, K, N), nb, X.device)
    md = _mask_bufs(M, K, X.device, M == 1) if mask_out else None
    ms = _mask_struct(md)
    L.check(lib.as_threshold_gemv(_ptr(X2), _dt(X2), M, K, _ptr(W), _dt(W), N, float(t), _ptr(Y), _dt(Y),
                                  flags, ctypes.byref(ms) if md else None, _ptr(ws), ws.numel(),
                                  _stream(X.device)), "as_threshold_gemv")
    out = Y[0] if squeeze else Y
    return (out, md) if mask_out else out


def as_dense_gemv(X: torch.Tensor, W: torch.Tensor, y_dtype=torch.float32, flags: int = 0,
                  Y: torch.Tensor | None = None):
    squeeze = X.dim() == 1
    X2 = X.reshape(1, -1) if squeeze else X
    _need_cuda(X2, W, Y)
    M, K = X2.shape
    N = W.shape[1]
    if Y is None:
        Y = torch.empty((M, N), dtype=y_dtype, device=X.device)
    lib = L.load()
    nb = lib.as_threshold_gemv_ws_size(M, K, N)
    ws = workspace(("gemv", M, K, N), nb, X.device)
    L.check(lib.as_dense_gemv(_ptr(X2), _dt(X2), M, K, _ptr(W), _dt(W), N, _ptr(Y), _dt(Y), flags,
                              _ptr(ws), ws.numel(), _stream(X.device)), "as_dense_gemv")
    return Y[0] if squeeze else Y


@dataclass
class MLPWeights:
    """THRESHOLD: w_gate_up [d_model, 2, d_ff], w_down [d_ff, d_model].
    NEURON_SET and GATE_SCORE: w_gate_up [d_ff, 3, d_model] (gate, up, down rows per
    neuron), w_down None."""
    w_gate_up: torch.Tensor
    w_down: Optional[torch.Tensor]
    mode: int = L.AS_MLP_THRESHOLD

    @property
    def d_model(self):
        return self.w_gate_up.shape[0] if self.mode == L.AS_MLP_THRESHOLD else self.w_gate_up.shape[2]

    @property
    def d_ff(self):
        return self.w_gate_up.shape[2] if self.mode == L.AS_MLP_THRESHOLD else self.w_gate_up.shape[0]

    def struct(self) -> L.ASMlpWeights:
        return L.ASMlpWeights(_ptr(self.w_gate_up), _ptr(self.w_down), _dt(self.w_gate_up),
                              self.d_model, self.d_ff)


def as_sparse_swiglu_mlp(X: torch.Tensor, w: MLPWeights, t_x: float = float("-inf"), t_h: float = float("-inf"),
                         neuron_idx: torch.Tensor | None = None, y_dtype=torch.float32, flags: int = 0,
                         debug: bool = False, events=None, Y: torch.Tensor | None = None):
    """Sparse SwiGLU MLP (THRESHOLD, NEURON_SET or GATE_SCORE per ``w.mode``; in
    GATE_SCORE ``t_h`` is the threshold on |silu(g)|).  With ``debug`` returns
    (Y, dict(h=..., x_mask=..., h_mask=..., a=...)) as the mode exports them."""
    squeeze = X.dim() == 1
    X2 = X.reshape(1, -1) if squeeze else X
    _need_cuda(X2, w.w_gate_up, w.w_down, neuron_idx, Y)
    M = X2.shape[0]
    d, f = w.d_model, w.d_ff
    if X2.shape[1] != d:
        raise ValueError(f"X has {X2.shape[1]} features, weights have d_model={d}")
    if Y is None:
        Y = torch.empty((M, d), dtype=y_dtype, device=X.device)
    lib = L.load()
    ws_ = w.struct()
    nb = lib.as_sparse_swiglu_mlp_ws_size(M, ctypes.byref(ws_), w.mode)
    ws = workspace(("mlp", w.mode, M, d, f), nb, X.device)
    n_active = 0 if neuron_idx is None else neuron_idx.numel()
    dbg = None
    dd = None
    if debug or events is not None:
        dbg = L.ASMlpDebug()
        if debug:
            dense = bool(flags & L.AS_FLAG_FORCE_DENSE)
            nh = f if (w.mode != L.AS_MLP_NEURON_SET) else (f if dense else n_active)
            dd = dict(h=torch.zeros((M, max(nh, 1)), dtype=torch.float32, device=X.device))
            dbg.h = _ptr(dd["h"])
            if w.mode == L.AS_MLP_THRESHOLD:
                dd["x_mask"] = _mask_bufs(M, d, X.device, M == 1)
                dd["h_mask"] = dict(bits=torch.zeros((M, (f + 63) // 64), dtype=torch.int64, device=X.device),
                                    nnz=torch.zeros(M, dtype=torch.int32, device=X.device))
                dbg.x_mask = _mask_struct(dd["x_mask"])
                dbg.h_mask = _mask_struct(dd["h_mask"])
            elif w.mode == L.AS_MLP_GATE_SCORE:
                dd["a"] = torch.zeros((M, f), dtype=torch.float32, device=X.device)
                dbg.a = _ptr(dd["a"])
                if not dense:
                    dd["h_mask"] = dict(bits=torch.zeros((M, (f + 63) // 64), dtype=torch.int64, device=X.device),
                                        nnz=torch.zeros(M, dtype=torch.int32, device=X.device))
                    dbg.h_mask = _mask_struct(dd["h_mask"])
        if events is not None:
            for i, e in enumerate(events):
                dbg.ev[i] = e.ev if e is not None else None
    L.check(lib.as_sparse_swiglu_mlp(_ptr(X2), _dt(X2), M, ctypes.byref(ws_), w.mode, float(t_x), float(t_h),
                                     _ptr(neuron_idx), n_active, _ptr(Y), _dt(Y), flags,
                                     ctypes.byref(dbg) if dbg is not None else None,
                                     _ptr(ws), ws.numel(), _stream(X.device)), "as_sparse_swiglu_mlp")
    out = Y[0] if squeeze else Y
    return (out, dd) if debug else out


def as_sparse_swiglu_mlp_noalloc(X: torch.Tensor, w: MLPWeights, Y: torch.Tensor, t_x: float = float("-inf"),
                                 t_h: float = float("-inf"), neuron_idx: torch.Tensor | None = None, flags: int = 0):
    """as_sparse_swiglu_mlp on the library's static per-device scratch (no workspace
    argument; the C call allocates nothing).  The caller passes the output Y."""
    X2 = X.reshape(1, -1) if X.dim() == 1 else X
    _need_cuda(X2, w.w_gate_up, w.w_down, neuron_idx, Y)
    ws_ = w.struct()
    n_active = 0 if neuron_idx is None else neuron_idx.numel()
    L.check(L.load().as_sparse_swiglu_mlp_noalloc(_ptr(X2), _dt(X2), X2.shape[0], ctypes.byref(ws_), w.mode,
                                                  float(t_x), float(t_h), _ptr(neuron_idx), n_active, _ptr(Y), _dt(Y),
                                                  flags, None, _stream(X.device)), "as_sparse_swiglu_mlp_noalloc")
    return Y


def as_topk_mask(score: torch.Tensor, k: int, prior: torch.Tensor | None = None, lam: float = 0.5,
                 mode: int | None = None, want_mask: bool = True, want_idx: bool = True):
    """Exact top-k per row (value mode, or the GLASS rank blend when ``prior`` is
    given).  score/prior: [rows, n] or [n] fp32.  Returns (mask words, idx)."""
    squeeze = score.dim() == 1
    s2 = score.reshape(1, -1) if squeeze else score
    p2 = None if prior is None else (prior.reshape(1, -1) if prior.dim() == 1 else prior)
    if p2 is not None and p2.shape != s2.shape:
        p2 = p2.expand_as(s2).contiguous()
    _need_cuda(s2, p2)
    if s2.dtype != torch.float32 or (p2 is not None and p2.dtype != torch.float32):
        raise TypeError("scores must be float32")
    rows, n = s2.shape
    if mode is None:
        mode = L.AS_TOPK_VALUE if p2 is None else L.AS_TOPK_RANK_BLEND
    dev = s2.device
    mask = torch.zeros((rows, (n + 63) // 64), dtype=torch.int64, device=dev) if want_mask else None
    idx = torch.zeros((rows, k), dtype=torch.int32, device=dev) if want_idx else None
    lib = L.load()
    nb = lib.as_topk_mask_ws_size(rows, n, mode)
    ws = workspace(("topk", rows, n, mode), nb, dev) if nb else None
    L.check(lib.as_topk_mask(_ptr(s2), _ptr(p2), rows, n, k, mode, float(lam), _ptr(mask), _ptr(idx),
                             _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)), "as_topk_mask")
    if squeeze:
        return (mask[0] if mask is not None else None), (idx[0] if idx is not None else None)
    return mask, idx


def as_moe_router(logits: torch.Tensor, top_k: int):
    """logits [T, E] fp32 -> (ids [T, top_k] int32 in descending-logit order, weights [T, top_k])."""
    _need_cuda(logits)
    T, E = logits.shape
    ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    wts = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    L.check(L.load().as_moe_router(_ptr(logits), T, E, top_k, _ptr(ids), _ptr(wts), _stream(logits.device)),
            "as_moe_router")
    return ids, wts


def as_moe_router_gemv(X: torch.Tensor, w_router: torch.Tensor, top_k: int):
    """Router logits X @ w_router and routing in one launch (T <= 8, E <= 512):
    returns (logits [T, E] fp32, ids [T, top_k] int32, weights [T, top_k])."""
    _need_cuda(X, w_router)
    T, d = X.shape
    E = w_router.shape[1]
    logits = torch.empty((T, E), dtype=torch.float32, device=X.device)
    ids = torch.empty((T, top_k), dtype=torch.int32, device=X.device)
    wts = torch.empty((T, top_k), dtype=torch.float32, device=X.device)
    lib = L.load()
    nb = lib.as_moe_router_gemv_ws_size(T, d, E)
    ws = workspace(("router", T, d, E), nb, X.device)
    L.check(lib.as_moe_router_gemv(_ptr(X), _dt(X), T, _ptr(w_router), _dt(w_router), d, E, top_k, _ptr(logits),
                                   _ptr(ids), _ptr(wts), _ptr(ws), ws.numel(), _stream(X.device)),
            "as_moe_router_gemv")
    return logits, ids, wts


@dataclass
class MoEWeights:
    """Routed experts (gate/up [E, d_ff_e, 2, d] neuron-major, down [E, d_ff_e, d]),
    router [d, E] and the dense shared expert (input-major gate/up [d, 2, d_ff_s],
    down [d_ff_s, d])."""
    w_gate_up: torch.Tensor
    w_down: torch.Tensor
    w_router: Optional[torch.Tensor] = None
    shared: Optional[MLPWeights] = None

    def struct(self) -> L.ASMoeWeights:
        E, f, _, d = self.w_gate_up.shape
        return L.ASMoeWeights(_ptr(self.w_gate_up), _ptr(self.w_down), _dt(self.w_gate_up), E, d, f)


def as_sparse_moe_expert(X: torch.Tensor, w: MoEWeights, ids: torch.Tensor, wts: torch.Tensor, keep_k: int,
                         y_dtype=torch.float32, flags: int = 0, Y: torch.Tensor | None = None, debug: bool = False,
                         y_ready: "L.HipEvent | None" = None):
    """Routed experts with intra-expert top-k; Y (+)= sum_j wts[t,j] * expert_{ids[t,j]}(X[t]).
    y_ready: event recorded after the producer of Y on another stream; only the down
    stage waits for it."""
    _need_cuda(X, w.w_gate_up, w.w_down, ids, wts, Y)
    T, d = X.shape
    top = ids.shape[1]
    E, f = w.w_gate_up.shape[0], w.w_gate_up.shape[1]
    if Y is None:
        Y = torch.empty((T, d), dtype=y_dtype, device=X.device)
    lib = L.load()
    st = w.struct()
    nb = lib.as_sparse_moe_expert_ws_size(T, top, ctypes.byref(st))
    ws = workspace(("moe", T, top, E, d, f), nb, X.device)
    h = keep = None
    if debug:
        h = torch.zeros((T, top, f), dtype=torch.float32, device=X.device)
        keep = torch.full((T, top, max(keep_k, 1)), -1, dtype=torch.int32, device=X.device)
    L.check(lib.as_sparse_moe_expert(_ptr(X), _dt(X), T, _ptr(ids), _ptr(wts), top, ctypes.byref(st), keep_k,
                                     _ptr(Y), _dt(Y), flags, _ptr(h), _ptr(keep),
                                     y_ready.ev if y_ready is not None else None, _ptr(ws), ws.numel(),
                                     _stream(X.device)), "as_sparse_moe_expert")
    return (Y, dict(h=h, keep=keep)) if debug else Y


def as_sparse_moe_expert_gate(X: torch.Tensor, w: MoEWeights, ids: torch.Tensor, wts: torch.Tensor, t_gate: float,
                              y_dtype=torch.float32, flags: int = 0, Y: torch.Tensor | None = None,
                              debug: bool = False, y_ready: "L.HipEvent | None" = None):
    """Routed experts under the gate-score keep rule (|silu(g)| > t_gate, up and
    down over the kept neurons); otherwise as as_sparse_moe_expert.  debug adds h
    and a ([T, top, d_ff_e] fp32)."""
    _need_cuda(X, w.w_gate_up, w.w_down, ids, wts, Y)
    T, d = X.shape
    top = ids.shape[1]
    E, f = w.w_gate_up.shape[0], w.w_gate_up.shape[1]
    if Y is None:
        Y = torch.empty((T, d), dtype=y_dtype, device=X.device)
    lib = L.load()
    st = w.struct()
    nb = lib.as_sparse_moe_expert_ws_size(T, top, ctypes.byref(st))
    ws = workspace(("moe", T, top, E, d, f), nb, X.device)
    h = a = None
    if debug:
        h = torch.zeros((T, top, f), dtype=torch.float32, device=X.device)
        a = torch.zeros((T, top, f), dtype=torch.float32, device=X.device)
    L.check(lib.as_sparse_moe_expert_gate(_ptr(X), _dt(X), T, _ptr(ids), _ptr(wts), top, ctypes.byref(st),
                                          float(t_gate), _ptr(Y), _dt(Y), flags, _ptr(h), _ptr(a),
                                          y_ready.ev if y_ready is not None else None, _ptr(ws), ws.numel(),
                                          _stream(X.device)), "as_sparse_moe_expert_gate")
    return (Y, dict(h=h, a=a)) if debug else Y


def _moe_layer_struct(w: MoEWeights) -> "L.ASMoeLayerWeights | None":
    if w.w_router is None or w.shared is None or w.w_router.dtype != torch.bfloat16:
        return None
    return L.ASMoeLayerWeights(_ptr(w.w_router), w.struct(), w.shared.struct())


def as_moe_layer(X: torch.Tensor, w: MoEWeights, top_k: int, keep_k: int, flags: int = 0, debug: bool = False):
    """The whole MoE layer on the current stream in three launches (C entry point
    as_moe_layer): router logits + routing beside the shared expert's gate/up, the
    routed gate/up beside the shared expert's down, then the routed down stage.
    Up to 8 tokens, bf16 weights; raises ASError (UNSUPPORTED) outside the limits.
    Returns Y [T, d] fp32 (and logits, ids, wts, h, keep when debug)."""
    _need_cuda(X, w.w_gate_up, w.w_down, w.w_router)
    T, d = X.shape
    E, f = w.w_gate_up.shape[0], w.w_gate_up.shape[1]
    lib = L.load()
    st = _moe_layer_struct(w)
    if st is None:
        raise ValueError("as_moe_layer: needs a bf16 router and a shared expert")
    nb = lib.as_moe_layer_ws_size(T, top_k, ctypes.byref(st))
    ws = workspace(("moe_layer", T, top_k, E, d, f, w.shared.d_ff), nb, X.device)
    Y = torch.empty((T, d), dtype=torch.float32, device=X.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=X.device)
    ids = torch.empty((T, top_k), dtype=torch.int32, device=X.device)
    wts = torch.empty((T, top_k), dtype=torch.float32, device=X.device)
    h = keep = None
    if debug:
        h = torch.zeros((T, top_k, f), dtype=torch.float32, device=X.device)
        keep = torch.full((T, top_k, max(keep_k, 1)), -1, dtype=torch.int32, device=X.device)
    L.check(lib.as_moe_layer(_ptr(X), _dt(X), T, ctypes.byref(st), top_k, keep_k, _ptr(Y), flags, _ptr(logits),
                             _ptr(ids), _ptr(wts), _ptr(h), _ptr(keep), _ptr(ws), ws.numel(), _stream(X.device)),
            "as_moe_layer")
    if debug:
        return Y, dict(logits=logits, ids=ids, wts=wts, h=h, keep=keep)
    return Y


def as_moe_layer_gate(X: torch.Tensor, w: MoEWeights, top_k: int, t_gate: float, flags: int = 0,
                      debug: bool = False):
    """as_moe_layer with the routed experts under the gate-score keep rule
    (|silu(g)| > t_gate).  Returns Y [T, d] fp32 (and logits, ids, wts, h, a when
    debug)."""
    _need_cuda(X, w.w_gate_up, w.w_down, w.w_router)
    T, d = X.shape
    E, f = w.w_gate_up.shape[0], w.w_gate_up.shape[1]
    lib = L.load()
    st = _moe_layer_struct(w)
    if st is None:
        raise ValueError("as_moe_layer_gate: needs a bf16 router and a shared expert")
    nb = lib.as_moe_layer_ws_size(T, top_k, ctypes.byref(st))
    ws = workspace(("moe_layer", T, top_k, E, d, f, w.shared.d_ff), nb, X.device)
    Y = torch.empty((T, d), dtype=torch.float32, device=X.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=X.device)
    ids = torch.empty((T, top_k), dtype=torch.int32, device=X.device)
    wts = torch.empty((T, top_k), dtype=torch.float32, device=X.device)
    h = a = None
    if debug:
        h = torch.zeros((T, top_k, f), dtype=torch.float32, device=X.device)
        a = torch.zeros((T, top_k, f), dtype=torch.float32, device=X.device)
    L.check(lib.as_moe_layer_gate(_ptr(X), _dt(X), T, ctypes.byref(st), top_k, float(t_gate), _ptr(Y), flags,
                                  _ptr(logits), _ptr(ids), _ptr(wts), _ptr(h), _ptr(a), _ptr(ws), ws.numel(),
                                  _stream(X.device)), "as_moe_layer_gate")
    if debug:
        return Y, dict(logits=logits, ids=ids, wts=wts, h=h, a=a)
    return Y


def moe_layer_one_stream_ok(X: torch.Tensor, w: MoEWeights, top_k: int, flags: int = 0) -> bool:
    """Whether as_moe_layer takes this call (shapes within its limits, bf16 weights)."""
    if flags & ~(L.AS_FLAG_FORCE_DENSE | L.AS_FLAG_ATOMIC_SPLITK):
        return False
    st = _moe_layer_struct(w)
    return st is not None and L.load().as_moe_layer_ws_size(X.shape[0], top_k, ctypes.byref(st)) > 0


_SIDE = {}


def _side_stream(device: torch.device) -> torch.cuda.Stream:
    """A second stream (default priority) per device, for work that can overlap."""
    k = str(device)
    if k not in _SIDE:
        _SIDE[k] = torch.cuda.Stream(device=device)
    return _SIDE[k]


_SIDE_EV = {}


def _side_event(device: torch.device) -> "L.HipEvent":
    """An event per device marking the end of the side stream's work."""
    k = str(device)
    if k not in _SIDE_EV:
        _SIDE_EV[k] = L.HipEvent()
    return _SIDE_EV[k]


def moe_layer(X: torch.Tensor, w: MoEWeights, top_k: int, keep_k: int, flags: int = 0, debug: bool = False,
              overlap: bool = True, one_stream: bool = True, t_gate: float | None = None):
    """One MoE layer: router logits (dense GEMV), router top-k + softmax, the dense
    shared expert, then the routed experts accumulated on top.  Where as_moe_layer
    takes the shapes (and `one_stream`), the layer is that one call: three launches
    on the current stream.  Otherwise it is composed from the separate entry points;
    with `overlap`, the shared expert then runs on a second stream while the router
    and the routed experts' gate/up stage run, and their down stage waits for it,
    since it accumulates into its output.  With `t_gate`, the routed experts keep
    the neurons with |silu(g)| > t_gate instead of the top keep_k (keep_k unused).
    Returns Y [T, d] fp32 (and intermediates when debug)."""
    if one_stream and moe_layer_one_stream_ok(X, w, top_k, flags):
        if t_gate is not None:
            return as_moe_layer_gate(X, w, top_k, t_gate, flags=flags, debug=debug)
        return as_moe_layer(X, w, top_k, keep_k, flags=flags, debug=debug)
    T, d = X.shape
    Y = torch.empty((T, d), dtype=torch.float32, device=X.device)
    cur = torch.cuda.current_stream(X.device)

    def shared():
        for t0 in range(0, T, 16):
            as_sparse_swiglu_mlp(X[t0:t0 + 16], w.shared, flags=L.AS_FLAG_FORCE_DENSE, Y=Y[t0:t0 + 16])

    side = _side_stream(X.device) if overlap else None
    ready = None
    if side is not None:
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            shared()
        ready = _side_event(X.device)
        ready.record(side.cuda_stream)
        Y.record_stream(side)
    E = w.w_router.shape[1]
    if T <= 8 and E <= 512 and E % 8 == 0 and top_k <= 64:
        logits, ids, wts = as_moe_router_gemv(X, w.w_router, top_k)
    else:
        logits = torch.empty((T, E), dtype=torch.float32, device=X.device)
        for t0 in range(0, T, 16):
            as_dense_gemv(X[t0:t0 + 16], w.w_router, Y=logits[t0:t0 + 16])
        ids, wts = as_moe_router(logits, top_k)
    if side is None:
        shared()
    # the routed experts' down stage waits for the shared expert (it accumulates
    # into Y); their grouping and gate/up stage overlap it
    if t_gate is not None:
        r = as_sparse_moe_expert_gate(X, w, ids, wts, t_gate, flags=flags | L.AS_FLAG_ACCUMULATE, Y=Y, debug=debug,
                                      y_ready=ready)
    else:
        r = as_sparse_moe_expert(X, w, ids, wts, keep_k, flags=flags | L.AS_FLAG_ACCUMULATE, Y=Y, debug=debug,
                                 y_ready=ready)
    if debug:
        return Y, dict(logits=logits, ids=ids, wts=wts, **r[1])
    return Y


def as_rmsnorm(X: torch.Tensor, eps: float = 1e-5, copy: bool = False):
    X2 = X.reshape(1, -1) if X.dim() == 1 else X
    _need_cuda(X2)
    rows, d = X2.shape
    Y = torch.empty((rows, d), dtype=torch.float32, device=X.device)
    C = torch.empty((rows, d), dtype=torch.float32, device=X.device) if copy else None
    L.check(L.load().as_rmsnorm(_ptr(X2), _dt(X2), rows, d, float(eps), _ptr(Y), _ptr(C), _stream(X.device)),
            "as_rmsnorm")
    Y = Y.reshape(X.shape)
    return (Y, C.reshape(X.shape)) if copy else Y


def as_gqa_decode_attention(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                            v_cache: torch.Tensor):
    """q [n_q, hd] fp32, k_new/v_new [n_kv, hd] fp32, caches [n_ctx, n_kv, hd] bf16 -> o [n_q, hd]."""
    _need_cuda(q, k_new, v_new, k_cache, v_cache)
    n_q, hd = q.shape
    n_ctx, n_kv, _ = k_cache.shape
    o = torch.empty((n_q, hd), dtype=torch.float32, device=q.device)
    lib = L.load()
    nb = lib.as_gqa_decode_attention_ws_size(n_ctx, n_q, n_kv, hd)
    ws = workspace(("attn", n_ctx, n_q, n_kv, hd), nb, q.device)
    L.check(lib.as_gqa_decode_attention(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                        _dt(k_cache), n_ctx, n_q, n_kv, hd, _ptr(o), _ptr(ws), ws.numel(),
                                        _stream(q.device)), "as_gqa_decode_attention")
    return o


@dataclass
class BlockWeights:
    """w_qkv [d, (n_q + 2 n_kv) hd], w_o [n_q hd, d], mlp (THRESHOLD layout)."""
    w_qkv: torch.Tensor
    w_o: torch.Tensor
    mlp: MLPWeights
    n_q: int = 32
    n_kv: int = 8
    head_dim: int = 128

    def struct(self) -> L.ASBlockWeights:
        return L.ASBlockWeights(_ptr(self.w_qkv), _ptr(self.w_o), self.mlp.struct(), self.n_q, self.n_kv,
                                self.head_dim)


def as_decoder_block(X: torch.Tensor, w: BlockWeights, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     t: dict, flags: int = 0, debug: bool = False, Y: torch.Tensor | None = None):
    """One decode token through a thresholded decoder block; t = dict(qkv=, o=, gate_up=, down=)."""
    X1 = X.reshape(-1)
    _need_cuda(X1, w.w_qkv, w.w_o, k_cache, v_cache, Y)
    d = X1.numel()
    if Y is None:
        Y = torch.empty(d, dtype=torch.float32, device=X.device)
    lib = L.load()
    st = w.struct()
    n_ctx = k_cache.shape[0]
    nb = lib.as_decoder_block_ws_size(ctypes.byref(st), n_ctx)
    ws = workspace(("block", d, w.mlp.d_ff, n_ctx, w.n_q, w.n_kv, w.head_dim), nb, X.device)
    th = L.ASBlockThresholds(float(t["qkv"]), float(t["o"]), float(t["gate_up"]), float(t["down"]))
    dd = None
    dbg = None
    if debug:
        nqkv = (w.n_q + 2 * w.n_kv) * w.head_dim
        no = w.n_q * w.head_dim
        z = lambda n: torch.zeros(n, dtype=torch.float32, device=X.device)  # noqa: E731
        dd = dict(xn=z(d), qkv=z(nqkv), o=z(no), h1=z(d), xn2=z(d), h=z(w.mlp.d_ff))
        masks = dict(qkv_in=_mask_bufs(1, d, X.device, True), o_in=_mask_bufs(1, no, X.device, True),
                     gate_up_in=_mask_bufs(1, d, X.device, True), down_in=_mask_bufs(1, w.mlp.d_ff, X.device, False))
        dd.update(masks)
        dbg = L.ASBlockDebug(*(_ptr(dd[k]) for k in ("xn", "qkv", "o", "h1", "xn2", "h")),
                             *(_mask_struct(masks[k]) for k in ("qkv_in", "o_in", "gate_up_in", "down_in")))
    L.check(lib.as_decoder_block(_ptr(X1), _dt(X1), ctypes.byref(st), _ptr(k_cache), _ptr(v_cache), n_ctx,
                                 ctypes.byref(th), _ptr(Y), flags, ctypes.byref(dbg) if dbg is not None else None,
                                 _ptr(ws), ws.numel(), _stream(X.device)), "as_decoder_block")
    return (Y, dd) if debug else Y


def calibrate_decoder_block(Xc: torch.Tensor, w: BlockWeights, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            p: float, flags: int = 0, keep_pools: bool = False):
    """Thresholds of one block's four thresholded inputs (qkv, o, gate_up, down) at
    target sparsity p from calibration vectors Xc [n, d] (the block's inputs).

    The pools are taken in input order, each with the thresholds of the earlier
    inputs applied (TEAL slides, method slide: thresholds from calibration data for
    the target sparsity); every pool and threshold is computed by the library
    (as_decoder_block's exported intermediates, as_calibrate_threshold).  Returns
    (thresholds, Y [n, d] fp32 = the block's outputs, which are the next block's
    calibration inputs, and the pools when keep_pools)."""
    inf = float("-inf")
    t = dict(qkv=inf, o=inf, gate_up=inf, down=inf)
    pools = {}
    for key, src in (("qkv", "xn"), ("o", "o"), ("gate_up", "xn2"), ("down", "h")):
        pool = torch.stack([as_decoder_block(Xc[i], w, k_cache, v_cache, t, flags=flags, debug=True)[1][src]
                            for i in range(Xc.shape[0])])
        t[key] = float(as_calibrate_threshold(pool, p).item())
        if keep_pools:
            pools[key] = pool
    Y = torch.stack([as_decoder_block(Xc[i], w, k_cache, v_cache, t, flags=flags) for i in range(Xc.shape[0])])
    return t, Y, (pools if keep_pools else None)


def as_glass_local_signal(X: torch.Tensor, w: MLPWeights) -> torch.Tensor:
    """Mean |h| of every FFN neuron over the prompt tokens X [P, d] (bf16); w neuron-major."""
    _need_cuda(X, w.w_gate_up)
    P = X.shape[0]
    local = torch.empty(w.d_ff, dtype=torch.float32, device=X.device)
    st = w.struct()
    L.check(L.load().as_glass_local_signal(_ptr(X), _dt(X), P, ctypes.byref(st), _ptr(local), _stream(X.device)),
            "as_glass_local_signal")
    return local


def as_bench_flush(buf: torch.Tensor):
    _need_cuda(buf)
    L.check(L.load().as_bench_flush(_ptr(buf), buf.numel() * buf.element_size(), _stream(buf.device)),
            "as_bench_flush")


def as_bench_read(buf: torch.Tensor, sink: torch.Tensor):
    _need_cuda(buf, sink)
    L.check(L.load().as_bench_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(buf.device)),
            "as_bench_read")


def unpack_bits(bits: torch.Tensor, n: int) -> torch.Tensor:
    """[M, words] int64 bitmask -> [M, n] bool (bit i%64 of word i//64)."""
    b = bits.cpu().view(torch.int64)
    shifts = torch.arange(64, dtype=torch.int64)
    m = ((b.unsqueeze(-1) >> shifts) & 1).bool().reshape(b.shape[0], -1)
    return m[:, :n]


class PreparedCall:
    """A library call with every argument resolved once, for tight launch loops
    (benchmarks, decode loops): calling it performs only the C call."""

    def __init__(self, fn, args, name, keep):
        self._fn, self._args, self._name, self._keep = fn, args, name, keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != L.AS_OK:
            L.check(st, self._name)


def prepare_sparse_swiglu_mlp(X: torch.Tensor, w: MLPWeights, t_x: float, t_h: float, Y: torch.Tensor,
                              neuron_idx: torch.Tensor | None = None, flags: int = 0, events=None) -> PreparedCall:
    X2 = X.reshape(1, -1) if X.dim() == 1 else X
    _need_cuda(X2, w.w_gate_up, w.w_down, neuron_idx, Y)
    M = X2.shape[0]
    lib = L.load()
    ws_ = w.struct()
    nb = lib.as_sparse_swiglu_mlp_ws_size(M, ctypes.byref(ws_), w.mode)
    ws = workspace(("mlp", w.mode, M, w.d_model, w.d_ff), nb, X.device)
    dbg = None
    if events is not None:
        dbg = L.ASMlpDebug()
        for i, e in enumerate(events):
            dbg.ev[i] = e.ev if e is not None else None
    n_active = 0 if neuron_idx is None else neuron_idx.numel()
    args = (_ptr(X2), _dt(X2), M, ctypes.byref(ws_), w.mode, ctypes.c_float(t_x), ctypes.c_float(t_h),
            _ptr(neuron_idx), n_active, _ptr(Y), _dt(Y), flags,
            ctypes.byref(dbg) if dbg is not None else None, _ptr(ws), ws.numel(), _stream(X.device))
    return PreparedCall(lib.as_sparse_swiglu_mlp, args, "as_sparse_swiglu_mlp", (ws_, dbg, ws, X2, Y))


def as_greedy_sparsity(err, weights, step: float, target: float):
    """Block-wise greedy sparsity levels (host arrays): ``err`` [n_blocks, n_levels]
    (error at sparsity level * step), ``weights`` [n_blocks]; returns int32 levels."""
    import numpy as np
    e = np.ascontiguousarray(err, dtype=np.float64)
    w = np.ascontiguousarray(weights, dtype=np.float64)
    if e.ndim != 2 or w.shape != (e.shape[0],):
        raise ValueError("err must be [n_blocks, n_levels] and weights [n_blocks]")
    out = np.zeros(e.shape[0], dtype=np.int32)
    lib = L.load()
    L.check(lib.as_greedy_sparsity(e.ctypes.data, e.shape[0], e.shape[1], w.ctypes.data, float(step), float(target),
                                   out.ctypes.data), "as_greedy_sparsity")
    return out


def as_threshold_gemv_i8(X: torch.Tensor, Wq: torch.Tensor, row_scale: torch.Tensor, t: float,
                         y_dtype=torch.float32, flags: int = 0, Y: torch.Tensor | None = None):
    """One token over int8 rows with a per-row scale:
    y = sum_{i: |x_i| > t} x_i * row_scale[i] * Wq[i, :].  X [K] or [1, K]; Wq [K, N] int8."""
    x = X.reshape(-1)
    _need_cuda(x, Wq, row_scale, Y)
    if Wq.dtype != torch.int8 or row_scale.dtype != torch.float32:
        raise ValueError("Wq must be int8 and row_scale float32")
    K, N = Wq.shape
    if Y is None:
        Y = torch.empty((N,), dtype=y_dtype, device=X.device)
    lib = L.load()
    nb = lib.as_threshold_gemv_i8_ws_size(K, N)
    ws = workspace(("gemv_i8", K, N), nb, X.device)
    L.check(lib.as_threshold_gemv_i8(_ptr(x), _dt(x), K, _ptr(Wq), _ptr(row_scale), N, float(t), _ptr(Y), _dt(Y),
                                     flags, _ptr(ws), ws.numel(), _stream(X.device)), "as_threshold_gemv_i8")
    return Y


def as_corrected_gxo(x: torch.Tensor, grad: torch.Tensor) -> torch.Tensor:
    """Corrected GxO attribution score per row (layer): grad*x + |x| * ||grad|| / 2."""
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    g2 = grad.reshape(x2.shape)
    _need_cuda(x2, g2)
    if x2.dtype != torch.float32 or g2.dtype != torch.float32:
        raise ValueError("x and grad must be float32")
    out = torch.empty_like(x2)
    L.check(L.load().as_corrected_gxo(_ptr(x2), _ptr(g2), x2.shape[0], x2.shape[1], _ptr(out), _stream(x.device)),
            "as_corrected_gxo")
    return out


def as_select_top_fraction(score: torch.Tensor, ar_num: int, ar_den: int):
    """Per-row top fraction ar_num/ar_den of the scores: (bitmask [rows, words], idx [rows, k])."""
    s2 = score.reshape(1, -1) if score.dim() == 1 else score
    _need_cuda(s2)
    rows, n = s2.shape
    lib = L.load()
    k = lib.as_top_fraction_count(n, int(ar_num), int(ar_den))
    if k < 0:
        raise ValueError(f"ratio {ar_num}/{ar_den} outside [0, 1]")
    mask = torch.zeros((rows, (n + 63) // 64), dtype=torch.int64, device=score.device)
    idx = torch.zeros((rows, max(k, 1)), dtype=torch.int32, device=score.device)
    L.check(lib.as_select_top_fraction(_ptr(s2), rows, n, int(ar_num), int(ar_den), _ptr(mask), _ptr(idx),
                                       _stream(score.device)), "as_select_top_fraction")
    return mask, idx[:, :k]


def as_head_masked_gemv(X: torch.Tensor, W: torch.Tensor, heads: torch.Tensor, n_heads: int, head_dim: int,
                        y_dtype=torch.float32, flags: int = 0, Y: torch.Tensor | None = None):
    """One token's output projection over the listed heads' row blocks of W."""
    x = X.reshape(-1)
    _need_cuda(x, W, heads, Y)
    N = W.shape[1]
    if Y is None:
        Y = torch.empty((N,), dtype=y_dtype, device=X.device)
    lib = L.load()
    nb = lib.as_head_masked_gemv_ws_size(n_heads, head_dim, N)
    ws = workspace(("head_gemv", n_heads, head_dim, N), nb, X.device)
    L.check(lib.as_head_masked_gemv(_ptr(x), _dt(x), n_heads, head_dim, _ptr(heads), heads.numel(), _ptr(W), _dt(W),
                                    N, _ptr(Y), _dt(Y), flags, _ptr(ws), ws.numel(), _stream(X.device)),
            "as_head_masked_gemv")
    return Y


def as_pack_neuron_set(w: MLPWeights, idx: torch.Tensor) -> MLPWeights:
    """Compact THRESHOLD-layout copy of the neurons idx (int32, device): gate/up
    [d_model, 2, k] and down [k, d_model]; run it with AS_FLAG_FORCE_DENSE for the
    static-set SwiGLU of a batch."""
    if w.mode != L.AS_MLP_THRESHOLD:
        raise ValueError("pack from THRESHOLD-layout weights")
    idx = idx.reshape(-1).contiguous()
    _need_cuda(w.w_gate_up, w.w_down, idx)
    k = idx.numel()
    gu = torch.empty((w.d_model, 2, k), dtype=w.w_gate_up.dtype, device=idx.device)
    dn = torch.empty((k, w.d_model), dtype=w.w_down.dtype, device=idx.device)
    ws_ = w.struct()
    L.check(L.load().as_pack_neuron_set(ctypes.byref(ws_), _ptr(idx), k, _ptr(gu), _ptr(dn), _stream(idx.device)),
            "as_pack_neuron_set")
    return MLPWeights(gu, dn, L.AS_MLP_THRESHOLD)
