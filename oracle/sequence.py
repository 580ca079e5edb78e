"""fp64 oracle: the sequence-parallel sum + LayerNorm (test infrastructure only).

Follows "Tensor Parallelism > Combining Column and Row Parallelism"
(mbrenndoerfer.com): the paragraph that names softmax and LayerNorm as
operations that reduce over the whole feature dimension, so they cannot be
split across GPUs by columns the way the weight matrices are; and FFN step 3
with the closing paragraph (the partials are summed, then the residual is
added).  The page gives no algorithm beyond that.  Reading taken: the rows
(tokens) are split instead -- each GPU sums only its block of rows of the t
partials plus the residual (the reduce-scatter half of the all-reduce),
applies LayerNorm to those full-width rows, and the blocks of all GPUs
together form the normalized matrix every GPU needs next (the all-gather
half).  Since both the sum and LayerNorm act row by row, that reaches the
unsharded result exactly (up to rounding order), so the oracle is written
unsharded: x = sum_i P_i + R, y = LayerNorm(x) row by row.

LayerNorm reading (the page names it only): the standard per-row form,
    y = (x - mean(x)) / sqrt(var(x) + eps) * gamma + beta,
mean and the biased variance taken over the row's features, eps added
inside the square root, gamma and beta per feature (gamma = 1 and beta = 0
when not given).
"""
from __future__ import annotations

import numpy as np

from .reduce import partial_reduce


def layernorm(x, gamma=None, beta=None, eps: float = 1e-5) -> np.ndarray:
    """LayerNorm over the last axis of x (rows are tokens), in float64."""
    x = np.asarray(x, np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mean) / np.sqrt(var + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, np.float64)
    if beta is not None:
        y = y + np.asarray(beta, np.float64)
    return y


def reduce_layernorm(partials, residual, gamma=None, beta=None, eps: float = 1e-5):
    """(x, y): x = sum_i partials[i] + residual (the residual stream after
    the sub-layer), y = LayerNorm(x) row by row; both float64."""
    x = partial_reduce(partials, residual)
    return x, layernorm(x, gamma, beta, eps)
