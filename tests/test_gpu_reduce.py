"""GPU parity of tp_partial_reduce (through the C ABI) against the oracle.

Bound used for fp32 accumulation: each of the t additions (t-1 partials and
the residual) rounds once to fp32, so per element
    |gpu - exact| <= t * 2^-24 * sum_i |term_i|     (fp32 output)
and a bf16 output adds one rounding of at most 2^-8 |exact| (unit roundoff
of an 8-bit significand).
"""
import numpy as np
import pytest
import torch

import oracle
from attention_shards_amd import synthetic as syn
from parity import empty, from_dev, log, to_dev

pytestmark = pytest.mark.gpu


def check_bound(got, parts, R, out_dtype):
    exact = oracle.partial_reduce(parts, R)
    mag = sum(np.abs(p) for p in parts) + (np.abs(R) if R is not None else 0)
    t = len(parts) + (1 if R is not None else 0)
    bound = t * 2.0 ** -24 * mag
    if out_dtype == syn.BF16:
        bound = bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(exact)
    assert np.all(np.abs(got - exact) <= bound + 1e-300)


@pytest.mark.parametrize("t,pdt,rdt,odt,rows,cols", [
    (4, syn.BF16, syn.BF16, syn.F32, 333, 264),
    (8, syn.BF16, syn.BF16, syn.BF16, 64, 4096),
    (3, syn.F32, syn.F32, syn.F32, 17, 8),
    (1, syn.F32, None, syn.BF16, 5, 1000 * 8),
    (13, syn.F32, syn.BF16, syn.F32, 100, 72),
    (8, syn.F32, syn.BF16, syn.F32, 37, 104),   # one chunk of 7 partials
    (7, syn.BF16, None, syn.F32, 33, 200),      # clamped chunk of 8
])
def test_reduce_random(gpu, t, pdt, rdt, odt, rows, cols):
    parts_h = [syn.normal_tensor(900 + t, k, (rows, cols), 0.5, pdt) for k in range(t)]
    R_h = syn.normal_tensor(900 + t, 99, (rows, cols), 1.0, rdt) if rdt else None
    out = empty((rows, cols), odt)
    gpu.tp_partial_reduce([to_dev(p, pdt) for p in parts_h],
                          to_dev(R_h, rdt) if rdt else None, out)
    torch.cuda.synchronize()
    parts = [syn.to_f64(p, pdt) for p in parts_h]
    R = syn.to_f64(R_h, rdt) if rdt else None
    check_bound(from_dev(out), parts, R, odt)


def test_reduce_small_integers_exact(gpu):
    rng = np.random.default_rng(5)
    parts = [rng.integers(-100, 100, size=(64, 64)).astype(np.float32) for _ in range(8)]
    R = rng.integers(-100, 100, size=(64, 64)).astype(np.float32)
    out = empty((64, 64), syn.F32)
    gpu.tp_partial_reduce([to_dev(p, syn.F32) for p in parts], to_dev(R, syn.F32), out)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(out), oracle.partial_reduce(parts, R))


def test_reduce_copy_and_in_place(gpu):
    p = torch.randn(40, 64, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(p)
    gpu.tp_partial_reduce([p], None, out)
    torch.cuda.synchronize()
    assert torch.equal(out, p)                      # t=1, no residual: copy
    a = torch.randn(40, 64, device="cuda")
    b = torch.randn(40, 64, device="cuda")
    r = torch.randn(40, 64, device="cuda")
    r0 = from_dev(r)
    gpu.tp_partial_reduce([a, b], r, r)             # out is the residual
    torch.cuda.synchronize()
    check_bound(from_dev(r), [from_dev(a), from_dev(b)], r0, syn.F32)
    a2 = a.clone()
    gpu.tp_partial_reduce([a2, b], None, a2)        # out is partials[0]
    torch.cuda.synchronize()
    assert torch.equal(a2, a + b)


def test_reduce_layer_shape_sampled(gpu):
    """t=4 bf16 partials [8192, 12288] + bf16 residual -> fp32 out; 256 rows."""
    rows, cols, t = 8192, 12288, 4
    parts_h = [syn.normal_tensor(55, k, (rows, cols), 0.5, syn.BF16) for k in range(t)]
    R_h = syn.normal_tensor(55, 9, (rows, cols), 1.0, syn.BF16)
    out = empty((rows, cols), syn.F32)
    gpu.tp_partial_reduce([to_dev(p, syn.BF16) for p in parts_h], to_dev(R_h, syn.BF16), out)
    torch.cuda.synchronize()
    sel = syn.sample_rows(55, rows, 256)
    got = from_dev(out[torch.from_numpy(sel).cuda()])
    check_bound(got, [syn.to_f64(p[sel], syn.BF16) for p in parts_h],
                syn.to_f64(R_h[sel], syn.BF16), syn.F32)
    log("reduce t=4 [8192,12288] sampled rows within the fp32 bound")


@pytest.mark.parametrize("t,pdt,odt,rows,cols,nslices", [
    (8, syn.BF16, syn.F32, 1000, 264, 8),    # 1000 = 8 x 125
    (8, syn.BF16, syn.BF16, 1003, 64, 3),    # ragged: blocks of 335, 334, 334 rows
    (4, syn.F32, syn.F32, 5, 16, 8),         # more slices than rows: 3 empty blocks
])
def test_reduce_slices_tile_the_full_reduce(gpu, t, pdt, odt, rows, cols, nslices):
    """The row blocks of all slices, each written by its own call into an
    output pre-filled with NaN, equal the full reduce bit for bit; a single
    call writes only its own rows; one block against the oracle's bound."""
    parts_h = [syn.normal_tensor(950 + t, k, (rows, cols), 0.5, pdt) for k in range(t)]
    R_h = syn.normal_tensor(950 + t, 99, (rows, cols), 1.0, syn.BF16)
    parts = [to_dev(p, pdt) for p in parts_h]
    R = to_dev(R_h, syn.BF16)
    full = empty((rows, cols), odt)
    gpu.tp_partial_reduce(parts, R, full)
    sliced = empty((rows, cols), odt).fill_(float("nan"))
    for s in range(nslices):
        gpu.tp_partial_reduce_slice(parts, R, sliced, s, nslices)
    one = empty((rows, cols), odt).fill_(float("nan"))
    s1 = nslices // 2
    gpu.tp_partial_reduce_slice(parts, R, one, s1, nslices)
    torch.cuda.synchronize()
    assert torch.equal(sliced, full)
    base, extra = divmod(rows, nslices)
    r0 = s1 * base + min(s1, extra)
    r1 = r0 + base + (1 if s1 < extra else 0)
    assert torch.equal(one[r0:r1], full[r0:r1])
    assert torch.isnan(one[:r0]).all() and torch.isnan(one[r1:]).all()
    log(f"reduce slices t={t} rows={rows} nslices={nslices}: block {s1} = rows [{r0}, {r1})")
    if r1 > r0:
        check_bound(from_dev(one[r0:r1]), [syn.to_f64(p[r0:r1], pdt) for p in parts_h],
                    syn.to_f64(R_h[r0:r1], syn.BF16), odt)


def test_reduce_bf16_output_is_rne(gpu):
    """One fp32 partial, no residual, bf16 output is a pure conversion: it
    equals round-to-nearest-even on the host bit for bit (ties included)."""
    rng = np.random.default_rng(12)
    p = rng.standard_normal((64, 256)).astype(np.float32)
    # exact ties: bit patterns ending in 0x8000 round to even
    p.view(np.uint32)[0, :64] = (p.view(np.uint32)[0, :64] & 0xFFFF0000) | 0x8000
    out = empty((64, 256), syn.BF16)
    gpu.tp_partial_reduce([to_dev(p, syn.F32)], None, out)
    torch.cuda.synchronize()
    got = from_dev(out).astype(np.float32)
    host = syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(p))
    assert np.array_equal(got.view(np.uint32), host.view(np.uint32))
