"""GPU parity of tp_sp_reduce_layernorm (through the C ABI) against the fp64
oracle: a block of rows of x = sum of partials + residual and
y = LayerNorm(x) per row (the sequence-parallel variant of the sum for the
operations that reduce over all features)."""
import numpy as np
import pytest
import torch

import oracle
from attention_shards_amd import synthetic as syn
from parity import TOL_F32, empty, from_dev, log, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _inputs(seed, t, rows, cols, pdt, rdt, affine):
    parts = [syn.normal_tensor(seed, k, (rows, cols), 0.5, pdt) for k in range(t)]
    R = syn.normal_tensor(seed, 90, (rows, cols), 1.0, rdt) if rdt else None
    g = b = None
    if affine:
        g = 1.0 + syn.normal_tensor(seed, 91, (cols,), 0.1, syn.F32)
        b = syn.normal_tensor(seed, 92, (cols,), 0.1, syn.F32)
    return parts, R, g, b


def _reference(parts, R, g, b, pdt, rdt, eps):
    P = [syn.to_f64(p, pdt) for p in parts]
    Rf = syn.to_f64(R, rdt) if R is not None else None
    return oracle.reduce_layernorm(P, Rf, g, b, eps), P, Rf


def _run(gpu, parts, R, g, b, pdt, rdt, xdt, ydt, eps, slice_of=(0, 1)):
    rows, cols = parts[0].shape
    dp = [to_dev(p, pdt) for p in parts]
    dR = to_dev(R, rdt) if R is not None else None
    X = empty((rows, cols), xdt) if xdt else None
    Y = empty((rows, cols), ydt)
    dg = torch.from_numpy(np.ascontiguousarray(g)).cuda() if g is not None else None
    db = torch.from_numpy(np.ascontiguousarray(b)).cuda() if b is not None else None
    if slice_of == "all":
        t = len(parts)
        for j in range(t):
            gpu.tp_sp_reduce_layernorm(dp, dR, X, Y, dg, db, eps, slice_of=(j, t))
    else:
        gpu.tp_sp_reduce_layernorm(dp, dR, X, Y, dg, db, eps, slice_of=slice_of)
    torch.cuda.synchronize()
    return (from_dev(X) if X is not None else None), from_dev(Y)


@pytest.mark.parametrize("t,rows,cols,pdt,rdt,xdt,ydt,affine", [
    (3, 37, 72, syn.BF16, syn.BF16, syn.F32, syn.F32, True),
    (4, 300, 12288, syn.BF16, syn.BF16, syn.F32, syn.F32, True),
    (2, 64, 32768, syn.F32, syn.F32, syn.F32, syn.F32, False),    # widest row (8 groups per thread)
    (4, 40, 20000, syn.BF16, syn.BF16, syn.F32, syn.BF16, True),  # 6 groups per thread, ragged
    (5, 33, 14000, syn.BF16, syn.F32, syn.F32, syn.F32, True),    # 4 groups per thread, ragged
    (2, 16, 8192, syn.F32, syn.BF16, syn.BF16, syn.F32, False),   # 2 groups per thread
    (1, 5, 8, syn.F32, None, None, syn.F32, True),                # one group per row
    (8, 129, 4104, syn.BF16, syn.F32, syn.BF16, syn.F32, True),   # ragged groups per thread
])
def test_reduce_layernorm(gpu, t, rows, cols, pdt, rdt, xdt, ydt, affine):
    eps = 1e-5
    parts, R, g, b = _inputs(1000 + cols, t, rows, cols, pdt, rdt, affine)
    (x_ref, y_ref), P, Rf = _reference(parts, R, g, b, pdt, rdt, eps)
    x, y = _run(gpu, parts, R, g, b, pdt, rdt, xdt, ydt, eps)
    ey = rel_err(y, y_ref)
    log(f"sp t={t} [{rows},{cols}] p={pdt} r={rdt} x={xdt} y={ydt}: LayerNorm err {ey:.2e}")
    if ydt == syn.BF16:
        # one rounding to bf16 (2^-8 relative) on top of an fp32-accurate value
        assert np.all(np.abs(y - y_ref) <= 2.0 ** -8 * np.abs(y_ref) + 1e-5 * (1 + np.abs(y_ref)))
    else:
        assert ey <= TOL_F32
    if x is not None:
        # the sum: t fp32 additions (plus the residual), then the x rounding
        mag = sum(np.abs(p) for p in P) + (np.abs(Rf) if Rf is not None else 0)
        n_add = t + (1 if Rf is not None else 0)
        bound = n_add * 2.0 ** -24 * mag
        if xdt == syn.BF16:
            bound = bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(x_ref)
        assert np.all(np.abs(x - x_ref) <= bound + 1e-300)


def test_bf16_layernorm_output_is_within_its_rounding(gpu):
    t, rows, cols, eps = 4, 200, 4096, 1e-5
    parts, R, g, b = _inputs(77, t, rows, cols, syn.BF16, syn.BF16, True)
    (_, y_ref), _, _ = _reference(parts, R, g, b, syn.BF16, syn.BF16, eps)
    _, y = _run(gpu, parts, R, g, b, syn.BF16, syn.BF16, None, syn.BF16, eps)
    # one rounding to bf16 (2^-8 relative) on top of an fp32-accurate value
    assert np.all(np.abs(y - y_ref) <= 2.0 ** -8 * np.abs(y_ref) + 1e-5 * (1 + np.abs(y_ref)))


@pytest.mark.parametrize("t,rows", [(4, 1003), (8, 5)])   # ragged blocks; rows < slices
def test_row_blocks_assemble_the_single_call(gpu, t, rows):
    """Every slice j of t writes its rows in place: the t calls together give
    the one-call result bit for bit (the all-gather is the shared buffer)."""
    cols, eps = 1024, 1e-5
    parts, R, g, b = _inputs(88 + rows, t, rows, cols, syn.BF16, syn.BF16, True)
    x1, y1 = _run(gpu, parts, R, g, b, syn.BF16, syn.BF16, syn.F32, syn.F32, eps)
    xs, ys = _run(gpu, parts, R, g, b, syn.BF16, syn.BF16, syn.F32, syn.F32, eps, "all")
    assert np.array_equal(x1, xs) and np.array_equal(y1, ys)


def test_x_out_may_be_the_residual(gpu):
    """x written over the residual buffer (same element size): each row is
    read in full before it is written."""
    t, rows, cols, eps = 2, 64, 2048, 1e-5
    parts, R, g, b = _inputs(99, t, rows, cols, syn.F32, syn.F32, False)
    (x_ref, y_ref), _, _ = _reference(parts, R, g, b, syn.F32, syn.F32, eps)
    dp = [to_dev(p, syn.F32) for p in parts]
    dR = to_dev(R, syn.F32)
    Y = empty((rows, cols), syn.F32)
    gpu.tp_sp_reduce_layernorm(dp, dR, dR, Y, None, None, eps)
    torch.cuda.synchronize()
    assert rel_err(from_dev(Y), y_ref) <= TOL_F32
    assert rel_err(from_dev(dR), x_ref) <= 1e-6


def test_layer_shape_t4_sampled(gpu):
    """The four-way layer shape: 4 bf16 partials [8192, 12288] + bf16
    residual, fp32 x and bf16 LayerNorm output, each of the 4 row blocks
    computed by its own call; 128 seeded rows against the oracle."""
    t, rows, cols, eps = 4, 8192, 12288, 1e-5
    parts, R, g, b = _inputs(5, t, rows, cols, syn.BF16, syn.BF16, True)
    x, y = _run(gpu, parts, R, g, b, syn.BF16, syn.BF16, syn.F32, syn.F32, eps, "all")
    sel = syn.sample_rows(5, rows, 128)
    (x_ref, y_ref), _, _ = _reference([p[sel] for p in parts], R[sel], g, b, syn.BF16,
                                      syn.BF16, eps)
    e = rel_err(y[sel], y_ref)
    log(f"sp layer shape t=4 [8192,12288] (128 rows): LayerNorm err {e:.2e}, "
        f"x err {rel_err(x[sel], x_ref):.2e}")
    assert e <= TOL_F32 and rel_err(x[sel], x_ref) <= 1e-6
