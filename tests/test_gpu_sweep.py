"""GPU parity over the whole hidden-size sweep: hidden 2048..22528 step 2048,
ffn = 4 hidden, t in {1, 2, 4, 8}, 2048 tokens, shard 0 of t, bf16 inputs,
fp32 output (the 44 points of the throughput-vs-hidden-size chart).

Inputs per hidden size come from the seeded generator with seed
300 + hidden/2048; every t slices the same full W1 and W2 (W1_0 = the first
4h/t columns, a zero-copy view; W2_0 = the first 4h/t rows).  16 seeded rows
per point (the first and the last included) are compared with the oracle:
an output row depends only on its own input row, so the sample is exact for
those rows.  The oracle runs once per hidden size as the partials of the
eight column blocks of width h/2; shard 0 of t is the sum of the first 8/t
of them (the shard-sum identity, pinned in the oracle tests).
"""
import numpy as np
import pytest
import torch

import oracle
from attention_shards_amd import synthetic as syn
from parity import TOL_BF16, empty, from_dev, log, rel_err, to_dev

pytestmark = pytest.mark.gpu

TOKENS = 2048
HIDDEN = list(range(2048, 22528 + 1, 2048))
POINTS = [(h, t) for h in HIDDEN for t in (1, 2, 4, 8)]

_cache = {}


def _point_data(h):
    """Device tensors, sampled rows and the eight oracle block partials of one
    hidden size (the previous hidden size's are dropped first)."""
    if h in _cache:
        return _cache[h]
    _cache.clear()
    torch.cuda.empty_cache()
    seed = 300 + h // 2048
    f = 4 * h
    d = syn.make_ffn_inputs(seed, TOKENS, h, f, syn.BF16)
    rows = syn.sample_rows(seed, TOKENS, 16)
    X = syn.to_f64(d["X"][rows], syn.BF16)
    blocks = []
    for j in range(8):
        c = syn.column_slice(f, j, 8)
        blocks.append(oracle.ffn_shard(X, syn.to_f64(d["W1"][:, c], syn.BF16),
                                       syn.to_f64(d["W2"][c, :], syn.BF16)))
    dev = dict(X=to_dev(d["X"], syn.BF16), W1=to_dev(d["W1"], syn.BF16),
               W2=to_dev(d["W2"], syn.BF16))
    del d
    _cache[h] = (dev, rows, blocks)
    return _cache[h]


@pytest.mark.parametrize("h,t", POINTS, ids=[f"h{h}-t{t}" for h, t in POINTS])
def test_sweep_point(gpu, h, t):
    dev, rows, blocks = _point_data(h)
    fs = 4 * h // t
    Y = empty((TOKENS, h), syn.F32)
    gpu.tp_ffn_shard(dev["X"], dev["W1"][:, :fs], dev["W2"][:fs], Y, 0, t)
    torch.cuda.synchronize()
    got = from_dev(Y[torch.from_numpy(rows).cuda()])
    ref = sum(blocks[:8 // t])
    e = rel_err(got, ref)
    log(f"sweep h={h} t={t} (16 rows): err {e:.4f}")
    assert np.isfinite(got).all()
    assert e <= TOL_BF16
    if (h, t) == POINTS[-1]:
        _cache.clear()
        torch.cuda.empty_cache()
