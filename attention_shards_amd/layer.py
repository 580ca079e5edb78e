"""A whole transformer layer of t-way tensor parallelism, run on one GPU.

The page "Tensor Parallelism > Combining Column and Row Parallelism"
(mbrenndoerfer.com, closing paragraph on attention) chains two sub-layers per
layer: attention, whose per-GPU partials are summed and then get the residual
added, and the FFN on that result, summed and given its residual in the same
way.  Here the t shards run one after another on one GPU through the C ABI
(tp_attn_shard, tp_ffn_shard), and tp_partial_reduce stands for each of the
two sums.  No normalisation sits between the sub-layers (the page names
LayerNorm as an operation that is not split; it is not part of this layer).

Streams: X (bf16 in) -> X1 = sum_i attn_i + X (fp32) -> bf16 copy of X1 as
the FFN input -> X2 = sum_i ffn_i + X1 (fp32; the residual is the fp32 X1).
"""
from __future__ import annotations

from . import binding as B


def layer_forward(X, Wqkv, Wo, W1, W2, batch: int, seq: int, n_heads: int,
                  head_dim: int, causal: bool = True, ffn_partial_dtype=None,
                  stream=None):
    """X: [batch*seq, h] bf16.  Wqkv, Wo, W1, W2: lists of the t shards'
    tensors (Wqkv[i] [h, 3*(n_heads/t)*head_dim], Wo[i] [(n_heads/t)*head_dim,
    h], W1[i] [h, f/t] (a view with a row stride is fine), W2[i] [f/t, h]).
    Returns (X1, X2), both fp32 [batch*seq, h]."""
    import torch
    t = len(Wqkv)
    if not (len(Wo) == len(W1) == len(W2) == t):
        raise ValueError("every weight list must hold the t shards")
    M, h = X.shape
    dev = X.device
    pdt = ffn_partial_dtype or torch.float32
    s = B._stream_of(stream, dev)
    # every tensor below is allocated, used and freed in the order of `s`
    with torch.cuda.device(dev), torch.cuda.stream(s):
        attn = [torch.empty(M, h, device=dev, dtype=torch.float32) for _ in range(t)]
        for i in range(t):
            B.tp_attn_shard(X, Wqkv[i], Wo[i], attn[i], batch, seq, n_heads, head_dim, i, t,
                            causal, stream=s)
        X1 = torch.empty(M, h, device=dev, dtype=torch.float32)
        B.tp_partial_reduce(attn, X, X1, stream=s)
        X1b = torch.empty(M, h, device=dev, dtype=torch.bfloat16)
        B.tp_partial_reduce([X1], None, X1b, stream=s)
        ffn = [torch.empty(M, h, device=dev, dtype=pdt) for _ in range(t)]
        for i in range(t):
            B.tp_ffn_shard(X1b, W1[i], W2[i], ffn[i], i, t, stream=s)
        X2 = torch.empty(M, h, device=dev, dtype=torch.float32)
        B.tp_partial_reduce(ffn, X1, X2, stream=s)
    return X1, X2
