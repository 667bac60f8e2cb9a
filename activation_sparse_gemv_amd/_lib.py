"""ctypes declarations of libactsparse's C ABI (include/actsparse.h).

Loading fails loudly: there is no fallback implementation of any entry point.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int, c_int64, c_size_t, c_uint, c_void_p, c_char_p

LIB_PATH = os.environ.get("ACTSPARSE_LIB",
                          os.path.join(os.path.dirname(os.path.abspath(__file__)), "libactsparse.so"))

AS_OK, AS_ERR_INVALID_ARG, AS_ERR_UNSUPPORTED, AS_ERR_WORKSPACE, AS_ERR_HIP = range(5)
AS_F16, AS_BF16, AS_F32, AS_I8 = 0, 1, 2, 3
AS_FLAG_ACCUMULATE = 1 << 0
AS_FLAG_ATOMIC_SPLITK = 1 << 1
AS_FLAG_NO_NT_LOADS = 1 << 2
AS_FLAG_FORCE_DENSE = 1 << 3
AS_FLAG_NO_FUSION = 1 << 4
AS_FLAG_AUTO = 1 << 5
AS_AUTO_DENSE_MIN_TOKENS = 8
AS_MLP_THRESHOLD, AS_MLP_NEURON_SET, AS_MLP_GATE_SCORE = 0, 1, 2
AS_TOPK_VALUE, AS_TOPK_RANK_BLEND = 0, 1


class ASMaskOut(ctypes.Structure):
    _fields_ = [("bits", c_void_p), ("idx", c_void_p), ("nnz", c_void_p)]


class ASMlpWeights(ctypes.Structure):
    _fields_ = [("w_gate_up", c_void_p), ("w_down", c_void_p), ("w_dt", c_int),
                ("d_model", c_int), ("d_ff", c_int)]


class ASMoeWeights(ctypes.Structure):
    _fields_ = [("w_gate_up", c_void_p), ("w_down", c_void_p), ("w_dt", c_int), ("n_experts", c_int),
                ("d_model", c_int), ("d_ff_e", c_int)]


class ASMoeLayerWeights(ctypes.Structure):
    _fields_ = [("w_router", c_void_p), ("experts", ASMoeWeights), ("shared", ASMlpWeights)]


class ASBlockWeights(ctypes.Structure):
    _fields_ = [("w_qkv", c_void_p), ("w_o", c_void_p), ("mlp", ASMlpWeights), ("n_q", c_int), ("n_kv", c_int),
                ("head_dim", c_int)]


class ASBlockThresholds(ctypes.Structure):
    _fields_ = [("qkv", c_float), ("o", c_float), ("gate_up", c_float), ("down", c_float)]


class ASBlockDebug(ctypes.Structure):
    _fields_ = [("xn", c_void_p), ("qkv", c_void_p), ("o", c_void_p), ("h1", c_void_p), ("xn2", c_void_p),
                ("h", c_void_p), ("qkv_in", ASMaskOut), ("o_in", ASMaskOut), ("gate_up_in", ASMaskOut),
                ("down_in", ASMaskOut)]


class ASMlpDebug(ctypes.Structure):
    _fields_ = [("h", c_void_p), ("x_mask", ASMaskOut), ("h_mask", ASMaskOut), ("ev", c_void_p * 3),
                ("a", c_void_p)]


# name -> (restype, argtypes); every symbol declared in include/actsparse.h
SIGNATURES = {
    "as_version": (c_int, []),
    "as_status_string": (c_char_p, [c_int]),
    "as_last_error": (c_char_p, []),
    "as_workspace_init": (c_int, [c_void_p, c_size_t, c_void_p]),
    "as_calibrate_threshold_ws_size": (c_size_t, [c_int64]),
    "as_calibrate_threshold": (c_int, [c_void_p, c_int, c_int64, c_int64, c_int64, c_void_p, c_void_p, c_size_t,
                                       c_void_p]),
    "as_threshold_gemv_ws_size": (c_size_t, [c_int, c_int, c_int]),
    "as_threshold_gemv": (c_int, [c_void_p, c_int, c_int, c_int, c_void_p, c_int, c_int, c_float,
                                  c_void_p, c_int, c_uint, POINTER(ASMaskOut), c_void_p, c_size_t, c_void_p]),
    "as_dense_gemv": (c_int, [c_void_p, c_int, c_int, c_int, c_void_p, c_int, c_int,
                              c_void_p, c_int, c_uint, c_void_p, c_size_t, c_void_p]),
    "as_sparse_swiglu_mlp_ws_size": (c_size_t, [c_int, POINTER(ASMlpWeights), c_int]),
    "as_sparse_swiglu_mlp": (c_int, [c_void_p, c_int, c_int, POINTER(ASMlpWeights), c_int, c_float, c_float,
                                     c_void_p, c_int, c_void_p, c_int, c_uint, POINTER(ASMlpDebug),
                                     c_void_p, c_size_t, c_void_p]),
    "as_sparse_swiglu_mlp_noalloc": (c_int, [c_void_p, c_int, c_int, POINTER(ASMlpWeights), c_int, c_float,
                                             c_float, c_void_p, c_int, c_void_p, c_int, c_uint, POINTER(ASMlpDebug),
                                             c_void_p]),
    "as_topk_mask_ws_size": (c_size_t, [c_int, c_int, c_int]),
    "as_topk_mask": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_float, c_void_p, c_void_p,
                             c_void_p, c_size_t, c_void_p]),
    "as_moe_router": (c_int, [c_void_p, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p]),
    "as_moe_router_gemv_ws_size": (c_size_t, [c_int, c_int, c_int]),
    "as_moe_router_gemv": (c_int, [c_void_p, c_int, c_int, c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_size_t, c_void_p]),
    "as_sparse_moe_expert_ws_size": (c_size_t, [c_int, c_int, POINTER(ASMoeWeights)]),
    "as_sparse_moe_expert": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_int, POINTER(ASMoeWeights),
                                     c_int, c_void_p, c_int, c_uint, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_size_t, c_void_p]),
    "as_sparse_moe_expert_gate": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_int, POINTER(ASMoeWeights),
                                          c_float, c_void_p, c_int, c_uint, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_size_t, c_void_p]),
    "as_moe_layer_gate": (c_int, [c_void_p, c_int, c_int, POINTER(ASMoeLayerWeights), c_int, c_float, c_void_p,
                                  c_uint, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                  c_void_p]),
    "as_moe_layer_ws_size": (c_size_t, [c_int, c_int, POINTER(ASMoeLayerWeights)]),
    "as_moe_layer": (c_int, [c_void_p, c_int, c_int, POINTER(ASMoeLayerWeights), c_int, c_int, c_void_p, c_uint,
                             c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "as_rmsnorm": (c_int, [c_void_p, c_int, c_int, c_int, c_float, c_void_p, c_void_p, c_void_p]),
    "as_gqa_decode_attention_ws_size": (c_size_t, [c_int, c_int, c_int, c_int]),
    "as_gqa_decode_attention": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                                        c_int, c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
    "as_decoder_block_ws_size": (c_size_t, [POINTER(ASBlockWeights), c_int]),
    "as_decoder_block": (c_int, [c_void_p, c_int, POINTER(ASBlockWeights), c_void_p, c_void_p, c_int,
                                 POINTER(ASBlockThresholds), c_void_p, c_uint, POINTER(ASBlockDebug), c_void_p,
                                 c_size_t, c_void_p]),
    "as_glass_local_signal": (c_int, [c_void_p, c_int, c_int, POINTER(ASMlpWeights), c_void_p, c_void_p]),
    "as_bench_flush": (c_int, [c_void_p, c_size_t, c_void_p]),
    "as_bench_read": (c_int, [c_void_p, c_size_t, c_void_p, c_void_p]),
    "as_greedy_sparsity": (c_int, [c_void_p, c_int, c_int, c_void_p, ctypes.c_double, ctypes.c_double, c_void_p]),
    "as_threshold_gemv_i8_ws_size": (c_size_t, [c_int, c_int]),
    "as_pack_neuron_set": (c_int, [POINTER(ASMlpWeights), c_void_p, c_int, c_void_p, c_void_p, c_void_p]),
    "as_corrected_gxo": (c_int, [c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p]),
    "as_top_fraction_count": (c_int, [c_int, c_int, c_int]),
    "as_select_top_fraction": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p]),
    "as_head_masked_gemv_ws_size": (c_size_t, [c_int, c_int, c_int]),
    "as_head_masked_gemv": (c_int, [c_void_p, c_int, c_int, c_int, c_void_p, c_int, c_void_p, c_int, c_int,
                                    c_void_p, c_int, c_uint, c_void_p, c_size_t, c_void_p]),
    "as_threshold_gemv_i8": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_int, c_float, c_void_p, c_int,
                                     c_uint, c_void_p, c_size_t, c_void_p]),
}

_lib = None


def load():
    """Load libactsparse.so (built in-tree by ``python -m activation_sparse_gemv_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libactsparse.so not found at {LIB_PATH}; build it with "
                          f"`python -m activation_sparse_gemv_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class ASError(RuntimeError):
    def __init__(self, status: int, fn: str):
        lib = load()
        self.status = status
        msg = lib.as_last_error().decode(errors="replace")
        super().__init__(f"{fn} -> {lib.as_status_string(status).decode()}: {msg}")


def check(status: int, fn: str):
    if status != AS_OK:
        raise ASError(status, fn)


# ---------------------------------------------------------------- HIP events
_hip = None


def hip():
    """libamdhip64 for raw HIP events (recorded on the stream the kernels run on)."""
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreate.argtypes = [POINTER(c_void_p)]
        h.hipEventRecord.argtypes = [c_void_p, c_void_p]
        h.hipEventSynchronize.argtypes = [c_void_p]
        h.hipEventElapsedTime.argtypes = [POINTER(c_float), c_void_p, c_void_p]
        h.hipEventDestroy.argtypes = [c_void_p]
        _hip = h
    return _hip


class HipEvent:
    def __init__(self):
        self.ev = c_void_p()
        r = hip().hipEventCreate(ctypes.byref(self.ev))
        if r != 0:
            raise RuntimeError(f"hipEventCreate failed ({r})")

    def record(self, stream: int):
        r = hip().hipEventRecord(self.ev, c_void_p(stream))
        if r != 0:
            raise RuntimeError(f"hipEventRecord failed ({r})")

    def elapsed_ms(self, later: "HipEvent") -> float:
        hip().hipEventSynchronize(later.ev)
        ms = c_float()
        r = hip().hipEventElapsedTime(ctypes.byref(ms), self.ev, later.ev)
        if r != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({r})")
        return ms.value

    def __del__(self):
        try:
            if self.ev:
                hip().hipEventDestroy(self.ev)
        except Exception:
            pass
