"""CPU oracle for the activation-sparse decode path (test infrastructure).

This package is the plain, slow, fp64 statement of what the GPU library must
compute.  It exists only to check the HIP path: the test suite, the smoke
check and the CPU-baseline leg of the benchmark may import it; the library and
its Python binding never do.  It shares no code with the HIP path: it imports
numpy (and, for a few special-case cross-checks in the tests, nothing else),
never the ``activation_sparse_gemv_amd`` package.

Every function works on float64 numpy arrays holding the exact values of the
bf16 / fp16 / fp32 inputs (those conversions are exact), and cites the passage
of the source pages it follows:

* TEAL slides  -- "【DL輪読会】Training-Free Activation Sparsity in Large
  Language Models" (reading-group slides on TEAL, ICLR 2025).
* GLASS summary -- "技術概要：GLASS – LLM の推論時スパース化のための
  グローバル・ローカル集約" (summary of arXiv 2508.14302).
* Intra-expert summary -- "Uncovering Intra-expert Activation Sparsity for
  Efficient Mixture-of-Expert Model Execution" (summary of arXiv 2605.08575).
* Attribution notes -- "Attribution-based Sparse Activation in Large Language
  Models" (MLSys 2026 talk notes).
* Glossary -- "アクティベーションスパーシティ（LLM）" (glossary page).

Parity status: every function here is pinned by a ``-m "not gpu"`` test against
the pages' worked example, closed forms, library routines on special cases,
exact integer arithmetic or brute force.  The decoder-block composition
(``block.decoder_block``) is pinned only through its parts and its dense
special case; the pages print no block-level output ("parity unpinned" for
end-to-end values against the pages).
"""
from . import teal, topk, moe, block, glass  # noqa: F401
