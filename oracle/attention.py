"""fp64 oracle: the attention shard (test infrastructure only; see oracle/__init__).

Follows "Tensor Parallelism > Combining Column and Row Parallelism"
(mbrenndoerfer.com), the multi-head attention paragraphs: the QKV projections
are column-parallel with each GPU holding the Q, K, V weights of its heads;
each head attends over the full sequence on its own; the concatenated head
outputs go through the row-parallel output projection, giving a partial sum.

Readings: contiguous head blocks per GPU; scale 1/sqrt(d); causal keeps keys
j <= s (diagonal included) and leaves the others out of the softmax; no
dropout, no positional encoding, no biases.
"""
from __future__ import annotations

import numpy as np


def _heads(n_heads: int, t: int, i: int):
    hs = n_heads // t
    return range(i * hs, (i + 1) * hs)


def attention_heads(Q: np.ndarray, K: np.ndarray, V: np.ndarray, batch: int,
                    seq: int, n_local: int, head_dim: int,
                    causal: bool = True) -> np.ndarray:
    """Per-head softmax attention, heads independent of one another.

    Q, K, V are [batch*seq, n_local*head_dim] with head j in columns
    [j*d, (j+1)*d).  For each sequence b and head j:
        s[r, c] = q_r . k_c / sqrt(d)           (c <= r when causal)
        p[r, :] = softmax over the kept keys of row r
        o_r     = sum_c p[r, c] v_c
    Returns O [batch*seq, n_local*head_dim] (heads concatenated in order).
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    O = np.zeros_like(Q)
    keep = np.ones((seq, seq), dtype=bool)
    if causal:
        keep = np.tril(keep)           # key index c <= query index r
    scale = 1.0 / np.sqrt(head_dim)
    for b in range(batch):
        rows = slice(b * seq, (b + 1) * seq)
        for j in range(n_local):
            c = slice(j * head_dim, (j + 1) * head_dim)
            s = (Q[rows, c] @ K[rows, c].T) * scale
            s_kept = np.where(keep, s, -np.inf)
            m = s_kept.max(axis=1, keepdims=True)
            e = np.where(keep, np.exp(s_kept - m), 0.0)
            p = e / e.sum(axis=1, keepdims=True)
            O[rows, c] = p @ V[rows, c]
    return O


def attn_shard(X, WQ, WK, WV, WO, batch: int, seq: int, n_heads: int,
               head_dim: int, i: int, t: int, causal: bool = True) -> np.ndarray:
    """GPU i's attention partial [batch*seq, h] from the FULL weights.

    W_Q, W_K, W_V are [h, n_heads*d] and W_o is [n_heads*d, h].  GPU i uses
    columns (resp. rows) of heads [i*n_heads/t, (i+1)*n_heads/t):
        Q_i = X W_Q[:, heads_i], K_i, V_i likewise
        O_i = attention over those heads
        Y_i = O_i W_o[heads_i, :]       (row-parallel output projection)
    """
    hs = n_heads // t
    cols = slice(i * hs * head_dim, (i + 1) * hs * head_dim)
    X = np.asarray(X, np.float64)
    Q = X @ np.asarray(WQ, np.float64)[:, cols]
    K = X @ np.asarray(WK, np.float64)[:, cols]
    V = X @ np.asarray(WV, np.float64)[:, cols]
    O = attention_heads(Q, K, V, batch, seq, hs, head_dim, causal)
    return O @ np.asarray(WO, np.float64)[cols, :]


def attn_full(X, WQ, WK, WV, WO, batch: int, seq: int, n_heads: int,
              head_dim: int, causal: bool = True) -> np.ndarray:
    """Unsharded multi-head attention output projection (t = 1)."""
    return attn_shard(X, WQ, WK, WV, WO, batch, seq, n_heads, head_dim, 0, 1,
                      causal)
