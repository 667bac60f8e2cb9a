"""The C-ABI library loads, exports every declared symbol and validates arguments
on the host (CPU only: no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

from activation_sparse_gemv_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "actsparse.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(as_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libactsparse.so is not built: run `python -m activation_sparse_gemv_amd.build`")
    return L.load()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"{n} declared in actsparse.h but not exported"
        assert n in L.SIGNATURES, f"{n} has no ctypes signature in the binding"
    for n in L.SIGNATURES:
        assert n in names, f"binding declares {n}, header does not"


def test_enum_values_match_the_header():
    """Every enumerator of actsparse.h (status codes, dtypes, flags, modes) has the same
    value in the binding, so a flag or code added on one side cannot drift."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    found = {}
    for name, expr in re.findall(r"\b(AS_[A-Z0-9_]+)\s*=\s*([0-9]+u?(?:\s*<<\s*[0-9]+)?)", src):
        m = re.fullmatch(r"([0-9]+)u?(?:\s*<<\s*([0-9]+))?", expr.strip())
        found[name] = int(m.group(1)) << int(m.group(2) or 0)
    assert {"AS_OK", "AS_ERR_HIP", "AS_BF16", "AS_FLAG_ATOMIC_SPLITK", "AS_TOPK_RANK_BLEND"} <= set(found)
    for name, v in found.items():
        assert getattr(L, name) == v, name


def test_version_and_strings(lib):
    assert lib.as_version() == 202
    assert lib.as_status_string(L.AS_ERR_WORKSPACE) == b"AS_ERR_WORKSPACE"


def _p(v=4096):
    return ctypes.c_void_p(v)


def test_gemv_validation(lib):
    st = lib.as_threshold_gemv(None, L.AS_BF16, 1, 64, _p(), L.AS_BF16, 64, 0.5, _p(), L.AS_F32, 0, None,
                               None, 0, None)
    assert st == L.AS_ERR_INVALID_ARG and b"NULL" in lib.as_last_error()
    st = lib.as_threshold_gemv(_p(), L.AS_BF16, 17, 64, _p(), L.AS_BF16, 64, 0.5, _p(), L.AS_F32, 0, None,
                               None, 0, None)
    assert st == L.AS_ERR_UNSUPPORTED
    st = lib.as_threshold_gemv(_p(), L.AS_BF16, 9, 64, _p(), L.AS_F16, 64, 0.5, _p(), L.AS_F32, 0, None,
                               None, 0, None)
    assert st == L.AS_ERR_UNSUPPORTED and b"MFMA" in lib.as_last_error()
    st = lib.as_threshold_gemv(_p(), L.AS_BF16, 1, 64, _p(), L.AS_BF16, 60, 0.5, _p(), L.AS_F32, 0, None,
                               None, 0, None)
    assert st == L.AS_ERR_INVALID_ARG
    st = lib.as_threshold_gemv(_p(), L.AS_BF16, 1, 64, _p(4100), L.AS_BF16, 64, 0.5, _p(), L.AS_F32, 0, None,
                               None, 0, None)
    assert st == L.AS_ERR_INVALID_ARG and b"aligned" in lib.as_last_error()
    st = lib.as_threshold_gemv(_p(), L.AS_F32, 1, 64, _p(), L.AS_F32, 64, 0.5, _p(), L.AS_F32, 0, None,
                               None, 0, None)
    assert st == L.AS_ERR_INVALID_ARG     # fp32 weights are not a supported storage type
    need = lib.as_threshold_gemv_ws_size(1, 4096, 4096)
    assert need > 0
    st = lib.as_threshold_gemv(_p(), L.AS_BF16, 1, 4096, _p(), L.AS_BF16, 4096, 0.5, _p(), L.AS_F32, 0, None,
                               _p(), need - 1, None)
    assert st == L.AS_ERR_WORKSPACE
    st = lib.as_dense_gemv(_p(), L.AS_BF16, 1, 4096, _p(), L.AS_BF16, 4096, _p(), L.AS_F32, 0, None, 0, None)
    assert st == L.AS_ERR_WORKSPACE
    # atomic split-K adds into fp32 only
    st = lib.as_threshold_gemv(_p(), L.AS_BF16, 1, 4096, _p(), L.AS_BF16, 4096, 0.5, _p(), L.AS_BF16,
                               L.AS_FLAG_ATOMIC_SPLITK, None, _p(), need, None)
    assert st == L.AS_ERR_UNSUPPORTED and b"fp32" in lib.as_last_error()


def test_mlp_validation(lib):
    w = L.ASMlpWeights(_p(), _p(), L.AS_BF16, 4096, 14336)
    need = lib.as_sparse_swiglu_mlp_ws_size(1, ctypes.byref(w), L.AS_MLP_THRESHOLD)
    assert need > 14336 * 4
    st = lib.as_sparse_swiglu_mlp(_p(), L.AS_BF16, 1, ctypes.byref(w), L.AS_MLP_THRESHOLD, 0.5, 0.5, None, 0,
                                  _p(), L.AS_F32, 0, None, _p(), need - 16, None)
    assert st == L.AS_ERR_WORKSPACE
    bad = L.ASMlpWeights(_p(), _p(), L.AS_BF16, 4096, 14300)
    st = lib.as_sparse_swiglu_mlp(_p(), L.AS_BF16, 1, ctypes.byref(bad), L.AS_MLP_THRESHOLD, 0.5, 0.5, None, 0,
                                  _p(), L.AS_F32, 0, None, _p(), 1 << 30, None)
    assert st == L.AS_ERR_INVALID_ARG and b"d_ff" in lib.as_last_error()
    st = lib.as_sparse_swiglu_mlp(_p(), L.AS_BF16, 1, ctypes.byref(w), L.AS_MLP_THRESHOLD, 0.5, 0.5, None, 0,
                                  _p(), L.AS_F16, L.AS_FLAG_ATOMIC_SPLITK, None, _p(), need, None)
    assert st == L.AS_ERR_UNSUPPORTED and b"fp32" in lib.as_last_error()
    nodown = L.ASMlpWeights(_p(), None, L.AS_BF16, 4096, 14336)
    st = lib.as_sparse_swiglu_mlp(_p(), L.AS_BF16, 1, ctypes.byref(nodown), L.AS_MLP_THRESHOLD, 0.5, 0.5, None,
                                  0, _p(), L.AS_F32, 0, None, _p(), 1 << 30, None)
    assert st == L.AS_ERR_INVALID_ARG
    st = lib.as_sparse_swiglu_mlp(_p(), L.AS_BF16, 1, ctypes.byref(nodown), L.AS_MLP_NEURON_SET, 0, 0, None,
                                  5, _p(), L.AS_F32, 0, None, _p(), 1 << 30, None)
    assert st == L.AS_ERR_INVALID_ARG and b"neuron_idx" in lib.as_last_error()
    st = lib.as_sparse_swiglu_mlp(_p(), L.AS_BF16, 1, ctypes.byref(nodown), L.AS_MLP_NEURON_SET, 0, 0, _p(),
                                  20000, _p(), L.AS_F32, 0, None, _p(), 1 << 30, None)
    assert st == L.AS_ERR_INVALID_ARG


def test_calibrate_validation(lib):
    """The target sparsity is an exact rational p_num / p_den in [0, 1]."""
    nb = lib.as_calibrate_threshold_ws_size(10)
    assert nb > 0
    cal = lib.as_calibrate_threshold
    assert cal(None, L.AS_F32, 10, 1, 2, _p(), _p(), nb, None) == L.AS_ERR_INVALID_ARG
    assert cal(_p(), L.AS_F32, 10, 11, 10, _p(), _p(), nb, None) == L.AS_ERR_INVALID_ARG    # p > 1
    assert cal(_p(), L.AS_F32, 10, -1, 10, _p(), _p(), nb, None) == L.AS_ERR_INVALID_ARG    # p < 0
    assert cal(_p(), L.AS_F32, 10, 1, 0, _p(), _p(), nb, None) == L.AS_ERR_INVALID_ARG      # p_den < 1
    assert cal(_p(), L.AS_F32, 0, 0, 1, _p(), _p(), nb, None) == L.AS_ERR_INVALID_ARG       # n < 1
    assert cal(_p(), L.AS_F32, 10, 1, 2, _p(), None, nb, None) == L.AS_ERR_WORKSPACE
    assert cal(_p(), L.AS_F32, 10, 1, 2, _p(), _p(), nb - 1, None) == L.AS_ERR_WORKSPACE


def test_atomic_splitk_rejects_overlapping_output(lib):
    """Without AS_FLAG_ACCUMULATE the atomic split-K paths clear Y before X is read, so
    an overlapping Y is refused on the host (nothing is launched)."""
    X = 1 << 20
    need = lib.as_threshold_gemv_ws_size(1, 4096, 4096)
    st = lib.as_threshold_gemv(_p(X), L.AS_BF16, 1, 4096, _p(), L.AS_BF16, 4096, 0.5, _p(X + 4096), L.AS_F32,
                               L.AS_FLAG_ATOMIC_SPLITK, None, _p(), need, None)
    assert st == L.AS_ERR_INVALID_ARG and b"apart from X" in lib.as_last_error()
    w = L.ASMlpWeights(_p(), _p(), L.AS_BF16, 4096, 14336)
    nm = lib.as_sparse_swiglu_mlp_ws_size(1, ctypes.byref(w), L.AS_MLP_THRESHOLD)
    st = lib.as_sparse_swiglu_mlp(_p(X), L.AS_F32, 1, ctypes.byref(w), L.AS_MLP_THRESHOLD, 0.5, 0.5, None, 0,
                                  _p(X), L.AS_F32, L.AS_FLAG_ATOMIC_SPLITK, None, _p(), nm, None)
    assert st == L.AS_ERR_INVALID_ARG and b"apart from X" in lib.as_last_error()
    mw = L.ASMoeWeights(_p(), _p(), L.AS_BF16, 128, 2048, 768)
    ne = lib.as_sparse_moe_expert_ws_size(1, 8, ctypes.byref(mw))
    st = lib.as_sparse_moe_expert(_p(X), L.AS_BF16, 1, _p(), _p(), 8, ctypes.byref(mw), 77, _p(X - 1024), L.AS_F32,
                                  L.AS_FLAG_ATOMIC_SPLITK, None, None, None, _p(), ne, None)
    assert st == L.AS_ERR_INVALID_ARG and b"apart from X" in lib.as_last_error()


def test_library_reads_no_environment():
    """The launch plans (and so the workspace carve-ups) depend on the shapes only:
    no library source reads an environment variable."""
    csrc = os.path.join(ROOT, "activation_sparse_gemv_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        src = open(os.path.join(csrc, f)).read()
        assert "getenv" not in src and "environ" not in src, f


def test_topk_moe_block_validation(lib):
    assert lib.as_topk_mask(None, None, 1, 10, 3, L.AS_TOPK_VALUE, 0.5, _p(), None, None, 0, None) == L.AS_ERR_INVALID_ARG
    assert lib.as_topk_mask(_p(), None, 1, 10, 11, L.AS_TOPK_VALUE, 0.5, _p(), None, None, 0, None) == L.AS_ERR_INVALID_ARG
    assert lib.as_topk_mask(_p(), None, 1, 10, 3, L.AS_TOPK_VALUE, 0.5, None, None, None, 0, None) == L.AS_ERR_INVALID_ARG
    assert lib.as_topk_mask(_p(), None, 1, 10, 3, L.AS_TOPK_RANK_BLEND, 0.5, _p(), None, _p(), 1 << 20, None) == L.AS_ERR_INVALID_ARG
    assert lib.as_topk_mask(_p(), _p(), 1, 10, 3, L.AS_TOPK_RANK_BLEND, 1.5, _p(), None, _p(), 1 << 20, None) == L.AS_ERR_INVALID_ARG
    assert lib.as_topk_mask(_p(), _p(), 1, 70000, 3, L.AS_TOPK_RANK_BLEND, 0.5, _p(), None, _p(), 1 << 30, None) == L.AS_ERR_UNSUPPORTED
    assert lib.as_topk_mask(_p(), _p(), 2, 100, 3, L.AS_TOPK_RANK_BLEND, 0.5, _p(), None, _p(), 16, None) == L.AS_ERR_WORKSPACE
    assert lib.as_topk_mask_ws_size(1, 14336, L.AS_TOPK_VALUE) == 0
    assert lib.as_moe_router(_p(), 1, 128, 0, _p(), _p(), None) == L.AS_ERR_INVALID_ARG
    assert lib.as_moe_router(_p(), 1, 2000, 8, _p(), _p(), None) == L.AS_ERR_INVALID_ARG
    mw = L.ASMoeWeights(_p(), _p(), L.AS_BF16, 128, 2048, 768)
    assert lib.as_sparse_moe_expert_ws_size(16, 8, ctypes.byref(mw)) > 0
    st = lib.as_sparse_moe_expert(_p(), L.AS_BF16, 64, _p(), _p(), 8, ctypes.byref(mw), 77, _p(), L.AS_F32, 0,
                                  None, None, None, _p(), 1 << 30, None)
    assert st == L.AS_ERR_INVALID_ARG          # T * top_k > 256
    st = lib.as_sparse_moe_expert(_p(), L.AS_BF16, 1, _p(), _p(), 8, ctypes.byref(mw), 800, _p(), L.AS_F32, 0,
                                  None, None, None, _p(), 1 << 30, None)
    assert st == L.AS_ERR_INVALID_ARG          # keep_k > d_ff_e
    assert lib.as_gqa_decode_attention(_p(), _p(), _p(), _p(), _p(), L.AS_F16, 16, 32, 8, 128, _p(), _p(), 1 << 30,
                                       None) == L.AS_ERR_UNSUPPORTED
    assert lib.as_gqa_decode_attention(_p(), _p(), _p(), _p(), _p(), L.AS_BF16, 16, 32, 3, 128, _p(), _p(), 1 << 30,
                                       None) == L.AS_ERR_INVALID_ARG
    assert lib.as_gqa_decode_attention(_p(), _p(), _p(), _p(), _p(), L.AS_BF16, 16, 64, 4, 128, _p(), _p(), 1 << 30,
                                       None) == L.AS_ERR_UNSUPPORTED       # group of 16 > 8
    assert lib.as_gqa_decode_attention(_p(), _p(), _p(), _p(), _p(), L.AS_BF16, 16, 32, 8, 64, _p(), _p(), 1 << 30,
                                       None) == L.AS_ERR_UNSUPPORTED       # head_dim != 128
    assert lib.as_rmsnorm(None, L.AS_F32, 1, 64, 1e-5, _p(), None, None) == L.AS_ERR_INVALID_ARG
    w = L.ASMlpWeights(_p(), None, L.AS_F16, 4096, 14336)
    assert lib.as_glass_local_signal(_p(), L.AS_BF16, 128, ctypes.byref(w), _p(), None) == L.AS_ERR_UNSUPPORTED
    bw = L.ASBlockWeights(_p(), _p(), L.ASMlpWeights(_p(), _p(), L.AS_BF16, 4096, 14336), 32, 8, 128)
    need = lib.as_decoder_block_ws_size(ctypes.byref(bw), 2048)
    assert need > 0
    th = L.ASBlockThresholds(0.5, 0.5, 0.5, 0.5)
    assert lib.as_decoder_block(_p(), L.AS_BF16, ctypes.byref(bw), _p(), _p(), 2048, ctypes.byref(th), _p(), 0,
                                None, _p(), need - 256, None) == L.AS_ERR_WORKSPACE
    # the down-input mask exports bits and nnz, never an index list
    dbg = L.ASBlockDebug()
    dbg.down_in = L.ASMaskOut(None, _p(), None)
    assert lib.as_decoder_block(_p(), L.AS_BF16, ctypes.byref(bw), _p(), _p(), 2048, ctypes.byref(th), _p(), 0,
                                ctypes.byref(dbg), _p(), need, None) == L.AS_ERR_UNSUPPORTED


def test_workspace_init_and_flush_validation(lib):
    assert lib.as_workspace_init(None, 64, None) == L.AS_ERR_INVALID_ARG
    assert lib.as_workspace_init(None, 0, None) == L.AS_OK
    assert lib.as_bench_flush(None, 64, None) == L.AS_ERR_INVALID_ARG
    assert lib.as_bench_read(None, 64, _p(), None) == L.AS_ERR_INVALID_ARG
    assert lib.as_bench_read(_p(), 60, _p(), None) == L.AS_ERR_INVALID_ARG      # not whole 16-byte vectors
    assert lib.as_bench_read(_p(4100), 64, _p(), None) == L.AS_ERR_INVALID_ARG  # misaligned
    assert lib.as_bench_read(None, 0, None, None) == L.AS_OK


def test_binding_refuses_cpu_tensors():
    import torch
    from activation_sparse_gemv_amd import api
    with pytest.raises(ValueError, match="device tensors"):
        api.as_threshold_gemv(torch.zeros(64, dtype=torch.bfloat16), torch.zeros(64, 64, dtype=torch.bfloat16), 0.5)


def test_moe_layer_limits_and_validation(lib):
    """as_moe_layer: the one-stream layer's shape limits (workspace size 0 outside
    them) and its argument checks, all returned before any launch."""
    mw = L.ASMoeWeights(_p(), _p(), L.AS_BF16, 128, 2048, 768)
    sw = L.ASMlpWeights(_p(), _p(), L.AS_BF16, 2048, 4096)
    lw = L.ASMoeLayerWeights(_p(), mw, sw)
    for T in (1, 2, 3, 4, 8):
        assert lib.as_moe_layer_ws_size(T, 8, ctypes.byref(lw)) > 0
    nb = lib.as_moe_layer_ws_size(1, 8, ctypes.byref(lw))
    assert lib.as_moe_layer_ws_size(9, 8, ctypes.byref(lw)) == 0                 # more than 8 tokens
    assert lib.as_moe_layer_ws_size(1, 33, ctypes.byref(lw)) == 0                # top_k above 32
    bad = [L.ASMoeLayerWeights(_p(), L.ASMoeWeights(_p(), _p(), L.AS_BF16, 100, 2048, 768), sw),   # E % 8
           L.ASMoeLayerWeights(_p(), L.ASMoeWeights(_p(), _p(), L.AS_BF16, 1024, 2048, 768), sw),  # E > 512
           L.ASMoeLayerWeights(_p(), L.ASMoeWeights(_p(), _p(), L.AS_F16, 128, 2048, 768),
                               L.ASMlpWeights(_p(), _p(), L.AS_F16, 2048, 4096)),                 # fp16
           L.ASMoeLayerWeights(_p(), mw, L.ASMlpWeights(_p(), _p(), L.AS_BF16, 1024, 4096))]      # d_model
    for b in bad:
        assert lib.as_moe_layer_ws_size(1, 8, ctypes.byref(b)) == 0

    def call(T=1, top=8, keep=77, flags=0, ws_bytes=1 << 30, logits=_p(), w=lw):
        return lib.as_moe_layer(_p(), L.AS_BF16, T, ctypes.byref(w), top, keep, _p(), flags, logits, _p(), _p(),
                                None, None, _p(), ws_bytes, None)
    assert call(T=9) == L.AS_ERR_UNSUPPORTED
    assert call(w=bad[0]) == L.AS_ERR_UNSUPPORTED
    assert call(keep=800) == L.AS_ERR_INVALID_ARG                 # keep_k > d_ff_e
    assert call(top=0) == L.AS_ERR_INVALID_ARG
    assert call(flags=L.AS_FLAG_NO_NT_LOADS) == L.AS_ERR_UNSUPPORTED
    assert call(logits=None) == L.AS_ERR_INVALID_ARG
    assert call(ws_bytes=nb - 1) == L.AS_ERR_WORKSPACE


def test_phase_timeline_only_in_the_opt_in_build(lib):
    """The phase-timeline entry point (include/actsparse_timeline.h) exists only in
    libactsparse_timeline.so; the product library's kernels carry no timeline code.
    The opt-in build, when present, rejects a NULL or too-small buffer."""
    for name in ("as_phase_timeline_arm", "as_attention_timeline_arm"):
        assert not hasattr(lib, name)
    tl_path = os.path.join(ROOT, "activation_sparse_gemv_amd", "libactsparse_timeline.so")
    if not os.path.exists(tl_path):
        pytest.skip("libactsparse_timeline.so not built (python -m activation_sparse_gemv_amd.build --timeline)")
    tl = ctypes.CDLL(tl_path)
    for name in ("as_phase_timeline_arm", "as_attention_timeline_arm"):
        f = getattr(tl, name)
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
        assert f(None, 1024) == L.AS_ERR_INVALID_ARG
        assert f(ctypes.c_void_p(16), 8) == L.AS_ERR_INVALID_ARG


def test_greedy_sparsity_matches_the_oracle(lib):
    """The C allocation takes the oracle's steps exactly (integer levels), on convex
    and on non-monotone curves, with ties and weights; bad arguments are rejected."""
    import numpy as np
    from oracle import greedy
    import activation_sparse_gemv_amd as asg
    rng = np.random.default_rng(12)
    for trial in range(40):
        nb, nl = int(rng.integers(1, 9)), int(rng.integers(1, 12))
        err = np.round(rng.standard_normal((nb, nl)).cumsum(axis=1), 1)     # ties and non-monotone steps
        w = rng.choice([1.0, 2.0, 0.5, 3.0], nb)
        step = float(rng.choice([0.05, 0.1, 0.125]))
        target = float(rng.uniform(0, 1))
        got = asg.as_greedy_sparsity(err, w, step, target)
        assert got.tolist() == greedy.greedy_allocate(err, w, step, target).tolist()
    e = np.zeros((2, 3))
    p = e.ctypes.data
    wv = np.ones(2)
    lv = np.zeros(2, dtype=np.int32)
    assert lib.as_greedy_sparsity(None, 2, 3, wv.ctypes.data, 0.1, 0.5, lv.ctypes.data) == L.AS_ERR_INVALID_ARG
    assert lib.as_greedy_sparsity(p, 0, 3, wv.ctypes.data, 0.1, 0.5, lv.ctypes.data) == L.AS_ERR_INVALID_ARG
    assert lib.as_greedy_sparsity(p, 2, 3, wv.ctypes.data, 0.0, 0.5, lv.ctypes.data) == L.AS_ERR_INVALID_ARG
    assert lib.as_greedy_sparsity(p, 2, 3, wv.ctypes.data, 0.1, 1.5, lv.ctypes.data) == L.AS_ERR_INVALID_ARG
    wbad = np.array([1.0, -1.0])
    assert lib.as_greedy_sparsity(p, 2, 3, wbad.ctypes.data, 0.1, 0.5, lv.ctypes.data) == L.AS_ERR_INVALID_ARG
    enan = np.array([[0.0, np.nan, 1.0], [0.0, 1.0, 2.0]])
    assert lib.as_greedy_sparsity(enan.ctypes.data, 2, 3, wv.ctypes.data, 0.1, 0.5, lv.ctypes.data) == L.AS_ERR_INVALID_ARG


def test_attribution_selection_validation(lib):
    assert lib.as_top_fraction_count(10, 3, 10) == 3
    assert lib.as_top_fraction_count(10, 31, 100) == 4
    assert lib.as_top_fraction_count(14336, 2, 5) == 5735
    assert lib.as_top_fraction_count(7, 0, 1) == 0 and lib.as_top_fraction_count(7, 1, 1) == 7
    assert lib.as_top_fraction_count(7, 2, 1) == -1 and lib.as_top_fraction_count(7, 1, 0) == -1
    assert lib.as_top_fraction_count(2**31 - 1, 2**31 - 2, 2**31 - 1) == 2**31 - 2
    assert lib.as_corrected_gxo(None, _p(), 1, 4, _p(), None) == L.AS_ERR_INVALID_ARG
    assert lib.as_corrected_gxo(_p(), _p(), 0, 4, _p(), None) == L.AS_ERR_INVALID_ARG
    assert lib.as_select_top_fraction(_p(), 1, 10, 3, 2, _p(), None, None) == L.AS_ERR_INVALID_ARG
    assert lib.as_select_top_fraction(_p(), 1, 10, 1, 2, None, None, None) == L.AS_ERR_INVALID_ARG
    assert lib.as_head_masked_gemv_ws_size(32, 128, 4096) > 32 * 128 * 4
    st = lib.as_head_masked_gemv(_p(), L.AS_BF16, 32, 128, _p(), 33, _p(), L.AS_BF16, 4096, _p(), L.AS_F32, 0,
                                 _p(), 1 << 30, None)
    assert st == L.AS_ERR_INVALID_ARG
    st = lib.as_head_masked_gemv(_p(), L.AS_BF16, 32, 128, _p(), 8, _p(), L.AS_BF16, 4096, _p(), L.AS_F32,
                                 L.AS_FLAG_FORCE_DENSE, _p(), 1 << 30, None)
    assert st == L.AS_ERR_UNSUPPORTED
