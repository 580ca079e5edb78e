"""fp64 oracle: the FFN shard (test infrastructure only; see oracle/__init__).

Follows "Tensor Parallelism > Combining Column and Row Parallelism"
(mbrenndoerfer.com), the two-layer FFN walk-through, steps 1 to 3.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erfc


def gelu(z: np.ndarray) -> np.ndarray:
    """Exact GeLU, z * Phi(z) = 0.5 * z * (1 + erf(z / sqrt(2))).

    The page applies "GeLU" element-wise between the two linear layers
    (FFN step 1 and the paragraph on where the nonlinearity fits); the exact
    erf form is the reading taken (not the tanh approximation).  Evaluated
    as 0.5 * z * erfc(-z / sqrt(2)), the same function (1 + erf(u) =
    erfc(-u)) without the cancellation of 1 + erf for z << 0, so the value
    is relatively accurate in the negative tail as well.
    """
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * erfc(-z / np.sqrt(2.0))


def column_parallel(X: np.ndarray, W1_i: np.ndarray) -> np.ndarray:
    """FFN step 1: Z_i = X W_{1,i}, then Zhat_i = GeLU(Z_i), applied locally.

    X is the full replicated input [M, h]; W1_i is this GPU's column shard
    [h, f/t].  Returns Zhat_i [M, f/t] in float64 (never rounded).
    """
    return gelu(np.asarray(X, np.float64) @ np.asarray(W1_i, np.float64))


def row_parallel(Zhat_i: np.ndarray, W2_i: np.ndarray) -> np.ndarray:
    """FFN step 2: Y_i = Zhat_i W_{2,i}, a partial sum over the full output.

    W2_i is this GPU's row shard [f/t, h], cut along W2's input dimension,
    the same dimension Zhat_i is cut along, so no gather sits in between.
    """
    return np.asarray(Zhat_i, np.float64) @ np.asarray(W2_i, np.float64)


def ffn_shard(X: np.ndarray, W1_i: np.ndarray, W2_i: np.ndarray) -> np.ndarray:
    """One GPU's FFN partial Y_i = GeLU(X W_{1,i}) W_{2,i} (steps 1 and 2)."""
    return row_parallel(column_parallel(X, W1_i), W2_i)


def ffn_full(X: np.ndarray, W1: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """The unsharded FFN GeLU(X W1) W2, which step 3's sum Y = sum_i Y_i
    must reproduce."""
    return ffn_shard(X, W1, W2)
