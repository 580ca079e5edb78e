"""CPU emulation of the attention shard's rounding points (test tooling).

The fp64 oracle never rounds an intermediate.  The GPU kernels round at
fixed points: the QKV projection's fp32 accumulators are stored in 16-bit
formats (single or as a hi/lo pair, hi = round(v), lo = round(v - hi)); the
softmax probabilities are rounded before the P.V product (the running
denominator sums the rounded values); O is stored for the output projection
in a 16-bit format (single or a hi/lo pair; the projection may read W_o
converted to fp16) or as an fp16 value plus its residual in bf8 (e5m2:
fp16's exponent range, 2 stored significand bits), the projection then
multiplying the fp16 part by W_o in fp16 and the bf8 part by W_o in bf8.
This module replays one such choice in numpy: every product is exact (fp64),
every rounding point is applied where the kernels apply it, and the softmax
runs online over 64-key tiles like the kernel.  Its error against the oracle
is what the choice costs, so a choice can be judged here, on the CPU, before
a kernel implements it.

Formats: "bf16", "fp16" (one 16-bit value), "bf16x2", "fp16x2" (hi/lo
pair), "f32" (no rounding beyond fp32); for O also "fp16+bf8" (hi fp16, lo
the fp32 residual rounded to bf8).  The score product with a pair on both
sides drops only lo.lo (three MFMA passes); a pair on one side and a single
value on the other takes two passes; singles one.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from attention_shards_amd import synthetic as syn

KT = 64  # keys per tile


@dataclasses.dataclass(frozen=True)
class Split:
    q: str = "bf16x2"
    k: str = "bf16x2"
    v: str = "fp16x2"
    p: str = "fp16"
    o: str = "bf16x2"
    wo: str = "bf16"   # W_o as stored ("bf16") or converted to fp16 ("fp16")
    # (O "fp16+bf8" fixes W_o: fp16 against O_hi, bf8 against O_lo)

    def name(self):
        return f"Q {self.q}, K {self.k}, V {self.v}, P {self.p}, O {self.o}, W_o {self.wo}"


# The split the GPU kernels implement: Q and K single fp16 (one score pass),
# V an fp16 hi/lo pair with fp16 P (two passes), O fp16 plus a bf8 residual.
KERNEL = Split(q="fp16", k="fp16", v="fp16x2", p="fp16", o="fp16+bf8")


def _f32(x):
    return np.asarray(x, np.float64).astype(np.float32)


def bf8(x):
    """Round to the nearest bf8 (OCP e5m2: 1 sign, 5 exponent bits of bias
    15, 2 stored significand bits; subnormals below 2^-14 in steps of 2^-16),
    ties to even.  Magnitudes are assumed below the largest finite value
    (57344)."""
    x = np.asarray(x, np.float64)
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    step = 2.0 ** (np.maximum(e, -14.0) - 2.0)
    return np.round(x / step) * step  # np.round: ties to even


def _single(x32, fmt):
    if fmt == "bf8":
        return bf8(x32)
    if fmt == "bf16":
        return syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(x32)).astype(np.float64)
    if fmt == "fp16":
        return x32.astype(np.float16).astype(np.float64)
    if fmt == "f32":
        return x32.astype(np.float64)
    raise ValueError(fmt)


def split_value(x, fmt):
    """(hi, lo) of fp32(x) in `fmt`; lo is 0 for single formats."""
    x32 = _f32(x)
    if fmt == "fp16+bf8":
        hi = _single(x32, "fp16")
        lo = bf8((x32.astype(np.float64) - hi).astype(np.float32))
        return hi, lo
    if fmt.endswith("x2"):
        base = fmt[:-2]
        hi = _single(x32, base)
        lo = _single((x32.astype(np.float64) - hi).astype(np.float32), base)
        return hi, lo
    return _single(x32, fmt), np.zeros_like(x32, dtype=np.float64)


def scores(qh, ql, kh, kl, q_pair, k_pair):
    s = qh @ kh.T
    if q_pair:
        s = s + ql @ kh.T
    if k_pair:
        s = s + qh @ kl.T
    return s


def attention_heads(Q, K, V, batch, seq, nl, d, causal, sp: Split):
    """Per-head attention with the kernels' rounding points; O before its
    own rounding (fp64 array)."""
    scale_log2 = np.log2(np.e) / np.sqrt(d)
    O = np.zeros_like(Q)
    qp, kp = sp.q.endswith("x2"), sp.k.endswith("x2")
    for b in range(batch):
        rows = slice(b * seq, (b + 1) * seq)
        for j in range(nl):
            c = slice(j * d, (j + 1) * d)
            qh, ql = split_value(Q[rows, c], sp.q)
            kh, kl = split_value(K[rows, c], sp.k)
            vh, vl = split_value(V[rows, c], sp.v)
            S = scores(qh, ql, kh, kl, qp, kp)
            m = np.full(seq, -np.inf)
            lsum = np.zeros(seq)
            o = np.zeros((seq, d))
            qi = np.arange(seq)[:, None]
            for k0 in range(0, seq, KT):
                kj = np.arange(k0, min(seq, k0 + KT))[None, :]
                st = S[:, k0:k0 + KT]
                keep = (kj <= qi) if causal else np.ones_like(st, dtype=bool)
                st = np.where(keep, st, -np.inf)
                m_new = np.maximum(m, st.max(axis=1) * scale_log2)
                m_use = np.where(np.isinf(m_new), 0.0, m_new)
                p = np.where(keep, np.exp2(st * scale_log2 - m_use[:, None]), 0.0)
                p = _single(_f32(p), sp.p)
                alpha = np.where(np.isinf(m), 0.0, np.exp2(m - m_use))
                lsum = lsum * alpha + p.sum(axis=1)
                o = o * alpha[:, None] + p @ (vh[k0:k0 + KT] + vl[k0:k0 + KT])
                m = m_new
            O[rows, c] = o / lsum[:, None]
    return O


def attn_shard(X, WQ, WK, WV, WO, batch, seq, n_heads, d, i, t, causal, sp: Split):
    """GPU i's attention partial with the rounding points of `sp` (inputs
    as fp64 arrays of the bf16 values, full weights as for the oracle)."""
    hs = n_heads // t
    cols = slice(i * hs * d, (i + 1) * hs * d)
    Q = X @ WQ[:, cols]
    K = X @ WK[:, cols]
    V = X @ WV[:, cols]
    O = attention_heads(Q, K, V, batch, seq, hs, d, causal, sp)
    oh, ol = split_value(O, sp.o)
    Wo = WO[cols, :]
    if sp.o == "fp16+bf8":
        return oh @ _single(_f32(Wo), "fp16") + ol @ bf8(Wo)
    if sp.wo == "fp16":
        Wo = _single(_f32(Wo), "fp16")
    return (oh + ol) @ Wo
