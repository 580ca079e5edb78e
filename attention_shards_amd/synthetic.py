"""Seeded synthetic inputs for the tensor-parallel shard path.

This module only *draws* inputs and converts their storage format.  It holds
none of the path's arithmetic, so both the fp64 oracle (under ``oracle/``)
and the GPU path can be fed the very same bytes from it.

Generator definition
--------------------
A tensor is identified by ``(seed, stream)``.  Its elements, flattened in
row-major order, are cut into blocks of ``BLOCK`` elements; block ``b`` is
drawn as

    numpy.random.Generator(PCG64(SeedSequence(seed, spawn_key=(stream, b))))
        .standard_normal(n_b, dtype=float32)

and multiplied by ``float32(sigma)``.  Blocks are independent, so they are
drawn on a thread pool and the result does not depend on the thread count.
bf16 tensors are the fp32 values rounded to nearest-even on the upper 16
bits and are kept as raw ``uint16`` bit patterns (numpy has no bf16 type).

Per-configuration recipes (which tensor gets which stream and sigma) are in
``make_ffn_inputs`` / ``make_attn_inputs``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK = 1 << 22

F32 = "f32"
BF16 = "bf16"


def _threads() -> int:
    n = os.environ.get("TP_SYNTH_THREADS")
    if n:
        return max(1, int(n))
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the bf16 bit patterns as uint16.  Finite inputs only (the
    generator never produces inf/nan).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of a stored tensor (bf16 bits or float32)."""
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def normal_tensor(seed: int, stream: int, shape, sigma: float,
                  dtype: str = BF16) -> np.ndarray:
    """Draw a seeded N(0, sigma^2) tensor (see the module docstring)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.uint16 if dtype == BF16 else np.float32)
    nblocks = (n + BLOCK - 1) // BLOCK
    s32 = np.float32(sigma)

    def fill(b: int) -> None:
        lo = b * BLOCK
        hi = min(n, lo + BLOCK)
        g = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence(seed, spawn_key=(stream, b))))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        v *= s32
        out[lo:hi] = f32_to_bf16_bits(v) if dtype == BF16 else v

    if nblocks <= 1:
        for b in range(nblocks):
            fill(b)
    else:
        with ThreadPoolExecutor(min(_threads(), nblocks)) as ex:
            list(ex.map(fill, range(nblocks)))
    return out.reshape(shape)


# ---------------------------------------------------------------------------
# Shard views (layout only: which slice of a full tensor a GPU holds)
# ---------------------------------------------------------------------------

def column_slice(f: int, i: int, t: int) -> slice:
    """Columns [i*f/t, (i+1)*f/t) of a full W1 (contiguous equal blocks)."""
    fs = f // t
    return slice(i * fs, (i + 1) * fs)


def head_slice(n_heads: int, head_dim: int, i: int, t: int) -> slice:
    """Columns of W_Q/W_K/W_V (rows of W_o) of heads [i*n_h/t, (i+1)*n_h/t)."""
    hs = n_heads // t
    return slice(i * hs * head_dim, (i + 1) * hs * head_dim)


def qkv_held_shard(WQ: np.ndarray, WK: np.ndarray, WV: np.ndarray,
                   n_heads: int, head_dim: int, i: int, t: int) -> np.ndarray:
    """The buffer GPU i holds for its heads: [W_Q,i | W_K,i | W_V,i]."""
    c = head_slice(n_heads, head_dim, i, t)
    return np.ascontiguousarray(np.concatenate([WQ[:, c], WK[:, c], WV[:, c]],
                                               axis=1))


# ---------------------------------------------------------------------------
# Recipes
# ---------------------------------------------------------------------------

SIGMA_ACT = 1.0
SIGMA_W = 0.02


def make_ffn_inputs(seed: int, tokens: int, hidden: int, ffn: int,
                    dtype: str = BF16, residual: bool = False) -> dict:
    """X[tokens,h] ~ N(0,1); full W1[h,f], W2[f,h] ~ N(0, 0.02^2);
    optional residual R[tokens,h] ~ N(0,1).  Streams 0,1,2,3 in that order."""
    d = {
        "X": normal_tensor(seed, 0, (tokens, hidden), SIGMA_ACT, dtype),
        "W1": normal_tensor(seed, 1, (hidden, ffn), SIGMA_W, dtype),
        "W2": normal_tensor(seed, 2, (ffn, hidden), SIGMA_W, dtype),
        "dtype": dtype,
    }
    if residual:
        d["R"] = normal_tensor(seed, 3, (tokens, hidden), SIGMA_ACT, dtype)
    return d


def make_attn_inputs(seed: int, batch: int, seq: int, hidden: int,
                     n_heads: int, head_dim: int, dtype: str = BF16) -> dict:
    """X[batch*seq,h] ~ N(0,1); full W_Q, W_K, W_V[h, n_h*d] and
    W_o[n_h*d, h] ~ N(0, 0.02^2).  Streams 0..4 in that order."""
    hd = n_heads * head_dim
    return {
        "X": normal_tensor(seed, 0, (batch * seq, hidden), SIGMA_ACT, dtype),
        "WQ": normal_tensor(seed, 1, (hidden, hd), SIGMA_W, dtype),
        "WK": normal_tensor(seed, 2, (hidden, hd), SIGMA_W, dtype),
        "WV": normal_tensor(seed, 3, (hidden, hd), SIGMA_W, dtype),
        "WO": normal_tensor(seed, 4, (hd, hidden), SIGMA_W, dtype),
        "dtype": dtype,
    }


def make_layer_inputs(seed: int, batch: int, seq: int, hidden: int,
                      n_heads: int, head_dim: int, ffn: int, dtype: str = BF16) -> dict:
    """One transformer layer: the attention inputs of make_attn_inputs
    (streams 0..4) plus the full FFN weights W1[h,f], W2[f,h] ~ N(0, 0.02^2)
    (streams 5, 6)."""
    d = make_attn_inputs(seed, batch, seq, hidden, n_heads, head_dim, dtype)
    d["W1"] = normal_tensor(seed, 5, (hidden, ffn), SIGMA_W, dtype)
    d["W2"] = normal_tensor(seed, 6, (ffn, hidden), SIGMA_W, dtype)
    return d


def sample_rows(seed: int, n_rows: int, count: int) -> np.ndarray:
    """Seeded, sorted subset of row indices that always holds 0 and n_rows-1."""
    if count >= n_rows:
        return np.arange(n_rows)
    g = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(seed, spawn_key=(99,))))
    mid = g.choice(np.arange(1, n_rows - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, n_rows - 1], mid]))
