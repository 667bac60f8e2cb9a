"""Block-wise greedy sparsity allocation (TEAL), in plain Python.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np


def greedy_allocate(err, weights, step: float, target: float):
    """Per-block sparsity levels under a model-wide sparsity target.

    TEAL slides, slide 10 (Block-wise Greedy Optimization): under an overall
    sparsity constraint, choose each block's sparsity to minimise the blocks'
    l2 activation errors: (1) start every block at sparsity 0; (2) measure, for
    each block, the error if its sparsity were raised a little; (3) raise the
    block whose error grows least; (4) repeat until the overall target is met.

    Readings: ``err[b][l]`` is block b's error at sparsity ``l * step`` (level l,
    l = 0 .. L-1, measured beforehand); the overall sparsity is the
    ``weights``-weighted mean of the block sparsities (weights: each block's
    share, e.g. its number of thresholded inputs); a step raises one block by one
    level; ties go to the smaller block index; a block at the last level is not
    raised.  Stops as soon as the overall sparsity reaches ``target`` (compared
    with a relative slack of 1e-12), or when every block is at the last level.
    Returns the int level of every block.
    """
    err = np.asarray(err, dtype=np.float64)
    w = np.asarray(weights, dtype=np.float64)
    nb, nl = err.shape
    lev = np.zeros(nb, dtype=np.int64)
    wsum = w.sum()

    def overall():
        return float((w * lev * step).sum() / wsum)

    while overall() < target * (1.0 - 1e-12):
        best, best_b = None, -1
        for b in range(nb):
            if lev[b] + 1 >= nl:
                continue
            inc = err[b, lev[b] + 1] - err[b, lev[b]]
            if best is None or inc < best:
                best, best_b = inc, b
        if best_b < 0:
            break
        lev[best_b] += 1
    return lev
