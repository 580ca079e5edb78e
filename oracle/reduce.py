"""fp64 oracle: sum of shard partials plus residual (test infrastructure only).

Follows "Tensor Parallelism > Combining Column and Row Parallelism"
(mbrenndoerfer.com): FFN step 3 (the partial sums Y_i are summed across GPUs,
Y = sum_i Y_i) and the closing paragraph on attention (residual connections
are added to the accumulated result).
"""
from __future__ import annotations

import numpy as np


def partial_reduce(partials, residual=None) -> np.ndarray:
    """out = (sum_i partials[i]) + residual, in float64; residual is added once."""
    acc = np.zeros_like(np.asarray(partials[0], dtype=np.float64))
    for p in partials:
        acc = acc + np.asarray(p, dtype=np.float64)
    if residual is not None:
        acc = acc + np.asarray(residual, dtype=np.float64)
    return acc
