"""The attention rounding-point emulator (tests/attn_rounding.py) on the
CPU: it is pinned to the oracle (no rounding -> the oracle's result), and it
records why the kernels round where they do.  Bar: max-abs error / RMS of
the oracle <= 2e-2 for bf16 inputs; a precision split is kept only if its
worst error over the attention test shapes stays within half of that.

Shapes: the GPU attention tests' (short and long, causal and full, ragged);
the long causal ones carry the largest max|Y| / RMS(Y) (row 0 of each
sequence is v_0 W_o itself) and decide the choice.
"""
import numpy as np
import pytest

import oracle
from attention_shards_amd import synthetic as syn
from attn_rounding import KERNEL, Split, attn_shard, bf8

HALF_BAR = 1e-2

# batch, seq, hidden, heads, t, i, causal (seeds as in the GPU tests: 40 + seq)
SHAPES = [
    (2, 100, 256, 4, 2, 1, True),
    (3, 65, 384, 6, 3, 2, True),
    (1, 513, 1024, 8, 4, 3, True),
    (1, 1100, 256, 2, 2, 1, True),
    (2, 1000, 512, 16, 2, 1, True),
    (1, 4000, 512, 8, 2, 0, True),
    (3, 40, 384, 6, 3, 2, False),
    (1, 1200, 256, 2, 2, 0, False),
]

_cache = {}


def _case(shape):
    if shape not in _cache:
        batch, seq, hidden, nh, t, i, causal = shape
        a = syn.make_attn_inputs(40 + seq, batch, seq, hidden, nh, 128)
        f = {k: syn.to_f64(a[k], syn.BF16) for k in ("X", "WQ", "WK", "WV", "WO")}
        ref = oracle.attn_shard(f["X"], f["WQ"], f["WK"], f["WV"], f["WO"], batch, seq, nh,
                                128, i, t, causal)
        _cache[shape] = (f, ref)
    return _cache[shape]


def emulated_error(shape, sp):
    batch, seq, hidden, nh, t, i, causal = shape
    f, ref = _case(shape)
    y = attn_shard(f["X"], f["WQ"], f["WK"], f["WV"], f["WO"], batch, seq, nh, 128, i, t,
                   causal, sp)
    return float(np.max(np.abs(y - ref)) / np.sqrt(np.mean(ref ** 2)))


def test_no_rounding_reproduces_the_oracle():
    exact = Split(q="f32", k="f32", v="f32", p="f32", o="f32", wo="bf16")
    for shape in [(2, 100, 256, 4, 2, 1, True), (3, 40, 384, 6, 3, 2, False)]:
        # fp32 storage of Q, K, V, P and O only: ~1e-7 relative
        assert emulated_error(shape, exact) < 2e-6


def test_rounding_only_o_to_bf16_costs_its_floor():
    """One rounding, of O to bf16, on the 4000-token causal shape: the error
    is what O's 8-bit significand allows after the output projection; it
    alone is above the bar, which is why O carries a residual."""
    sp = Split(q="f32", k="f32", v="f32", p="f32", o="bf16", wo="bf16")
    assert emulated_error((1, 4000, 512, 8, 2, 0, True), sp) > 2e-2


def test_bf8_rounding_closed_form():
    """bf8 (e5m2) values: 4 steps per binade (1, 1.25, 1.5, 1.75), ties to the
    even significand, subnormal steps of 2^-16 below 2^-14, sign symmetric."""
    x = np.array([1.0, 1.1, 1.125, 1.375, 1.625, 1.875, 3.0, 0.3, 57344.0,
                  2.0 ** -14, 2.0 ** -16, 2.0 ** -17, 3 * 2.0 ** -17, 2.0 ** -18, -1.1, 0.0])
    want = np.array([1.0, 1.0, 1.0, 1.5, 1.5, 2.0, 3.0, 0.3125, 57344.0,
                     2.0 ** -14, 2.0 ** -16, 0.0, 2.0 ** -15, 0.0, -1.0, 0.0])
    assert np.array_equal(bf8(x), want)
    # every value of [2^-14, 2): relative error at most 2^-3 (half of the
    # 2^-2 step relative to the binade's start)
    v = np.linspace(2.0 ** -14, 2.0, 100001)
    assert np.max(np.abs(bf8(v) - v) / v) <= 2.0 ** -3


@pytest.mark.parametrize("shape", SHAPES)
def test_kernel_split_within_half_the_bar(shape):
    """The kernels' split: Q and K single fp16 (one score pass), V as an fp16
    hi/lo pair with fp16 P (two passes), O as fp16 plus a bf8 residual (one
    fp16 pass against W_o in fp16, one bf8 pass of half the cost against
    W_o in bf8)."""
    e = emulated_error(shape, KERNEL)
    assert e <= HALF_BAR, (shape, e)


def test_fp16_bf8_o_matches_the_bf16_pair():
    """O as fp16 + bf8 residual costs what the bf16 hi/lo pair it replaced
    cost: the residual's 3 significant bits on top of fp16's 11 leave the
    worst shape within 10% of the pair's error (0.0050 vs 0.0048), where one
    fp16 value is 2.5x the pair's."""
    shape = (1, 4000, 512, 8, 2, 0, True)
    pair = emulated_error(shape, Split(q="fp16", k="fp16", o="bf16x2", wo="bf16"))
    mixed = emulated_error(shape, KERNEL)
    single = emulated_error(shape, Split(q="fp16", k="fp16", o="fp16", wo="fp16"))
    assert mixed <= 1.1 * pair, (mixed, pair)
    assert single > 2 * pair, (single, pair)


def test_single_fp16_o_or_v_exceeds_half_the_bar():
    """Cheaper splits rejected: O as one fp16 value (the output projection
    then reads W_o as fp16, exact for these weights) or V as one fp16 value
    leave the 4000-token causal shape above half the bar."""
    shape = (1, 4000, 512, 8, 2, 0, True)
    assert emulated_error(shape, Split(q="fp16", k="fp16", o="fp16", wo="fp16")) > HALF_BAR
    assert emulated_error(shape, Split(q="fp16", k="fp16", v="fp16")) > HALF_BAR
