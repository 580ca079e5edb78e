"""fp64 oracle: one transformer layer, unsharded (test infrastructure only).

Follows "Tensor Parallelism > Combining Column and Row Parallelism"
(mbrenndoerfer.com), the closing paragraph on attention: a layer runs the
attention sub-layer and then the FFN sub-layer; each ends in one sum of the
GPUs' partial results, after which the residual connection is added.  So a
layer has exactly two such sums.  LayerNorm, which the page names as an
operation that is not split across GPUs, is not part of this layer (no
normalisation is applied); neither are biases.

Because the sharded computation reaches the unsharded result exactly (up to
rounding order), the layer is written here unsharded, in float64:
    X1 = MHA(X) + X,     X2 = FFN(X1) + X1.
"""
from __future__ import annotations

import numpy as np

from .attention import attn_full
from .ffn import ffn_full


def layer(X, WQ, WK, WV, WO, W1, W2, batch: int, seq: int, n_heads: int,
          head_dim: int, causal: bool = True):
    """Returns (X1, X2): the stream after the attention sub-layer and after
    the FFN sub-layer, both [batch*seq, h] float64."""
    X = np.asarray(X, np.float64)
    X1 = attn_full(X, WQ, WK, WV, WO, batch, seq, n_heads, head_dim, causal) + X
    X2 = ffn_full(X1, W1, W2) + X1
    return X1, X2
