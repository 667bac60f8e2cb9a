"""libactsparse: activation-sparse GEMV for LLM decode on MI355X (gfx950).

The compute lives in the HIP library ``libactsparse.so`` (C ABI declared in
``include/actsparse.h``); ``api`` is a thin tensor-level binding with the same
entry-point names, and ``datagen`` draws the seeded synthetic inputs.
"""
from . import _lib  # noqa: F401
from .api import (  # noqa: F401
    BlockWeights, MLPWeights, MoEWeights, as_bench_flush, as_bench_read, as_calibrate_threshold, as_decoder_block, as_dense_gemv,
    as_greedy_sparsity, as_threshold_gemv_i8, as_corrected_gxo, as_select_top_fraction, as_head_masked_gemv,
    as_pack_neuron_set, as_sparse_moe_expert_gate, as_moe_layer_gate,
    as_glass_local_signal, as_gqa_decode_attention, as_moe_layer, as_moe_router, as_moe_router_gemv, as_rmsnorm,
    as_sparse_moe_expert, as_sparse_swiglu_mlp, as_threshold_gemv, as_topk_mask, as_version, calibrate_decoder_block,
    moe_layer, unpack_bits, workspace,
)
