"""GPU parity of tp_ffn_shard_reduce (FFN shard whose second GEMM adds the
pre-summed other partials and residual in its epilogue), through the C ABI.

Against the fp64 oracle: out = sum_j P_j + R with P_i = oracle.ffn_shard and
the peers' partials taken as given inputs.  Against the unfused calls in the
fused order (tp_partial_reduce of the other partials and R, tp_ffn_shard
with an fp32 Y_i, then tp_partial_reduce of that sum and Y_i): bitwise,
since both add the same fp32 values in the same order.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_shards_amd import synthetic as syn
from parity import TOL_BF16, TOL_F32, empty, from_dev, log, rel_err, to_dev

pytestmark = pytest.mark.gpu


def dev_inputs(d, i, t):
    dt = d["dtype"]
    f = d["W1"].shape[1]
    cols = syn.column_slice(f, i, t)
    X = to_dev(d["X"], dt)
    W1 = to_dev(d["W1"], dt)
    W2_i = to_dev(np.ascontiguousarray(d["W2"][cols, :]), dt)
    return X, W1[:, cols], W2_i


def peers_random(seed, t, M, h, dtype):
    """Arbitrary peer partials (the reduce does not care where they come from)."""
    return [syn.normal_tensor(seed, 10 + j, (M, h), 1.0, dtype) for j in range(t)]


def oracle_out(d, i, t, peers_np, pdt, R_np, rdt, rows=None):
    dt = d["dtype"]
    f = d["W1"].shape[1]
    cols = syn.column_slice(f, i, t)
    X = d["X"] if rows is None else d["X"][rows]
    Pi = oracle.ffn_shard(syn.to_f64(X, dt), syn.to_f64(d["W1"][:, cols], dt),
                          syn.to_f64(d["W2"][cols, :], dt))
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    parts = [Pi if j == i else syn.to_f64(sel(peers_np[j]), pdt) for j in range(t)]
    R = None if R_np is None else syn.to_f64(sel(R_np), rdt)
    return oracle.partial_reduce(parts, R)


@pytest.mark.parametrize("M,h,f,t,i,pdt,rdt,odt", [
    (300, 200, 3 * 424, 3, 1, syn.BF16, syn.BF16, syn.F32),   # ragged tiles
    (257, 264, 4 * 136, 4, 0, syn.F32, syn.F32, syn.F32),
    (130, 512, 2 * 512, 2, 1, syn.BF16, None, syn.BF16),      # no residual, bf16 out
    (64, 128, 512, 1, 0, syn.BF16, syn.BF16, syn.F32),        # t=1: out = P_0 + R
    (1000, 1000, 2 * 8200, 2, 1, syn.BF16, syn.BF16, syn.F32),  # GEMM2 splits K: S + partials
])
def test_fused_matches_oracle(gpu, M, h, f, t, i, pdt, rdt, odt):
    d = syn.make_ffn_inputs(700 + M, M, h, f, syn.BF16, residual=rdt is not None)
    X, W1_i, W2_i = dev_inputs(d, i, t)
    peers_np = peers_random(701 + M, t, M, h, pdt)
    peers = [None if j == i else to_dev(peers_np[j], pdt) for j in range(t)]
    R_np = None
    R = None
    if rdt is not None:
        R_np = d["R"] if rdt == syn.BF16 else syn.normal_tensor(702 + M, 0, (M, h), 1.0, syn.F32)
        R = to_dev(R_np, rdt)
    out = empty((M, h), odt)
    gpu.tp_ffn_shard_reduce(X, W1_i, W2_i, peers, R, out, i)
    torch.cuda.synchronize()
    ref = oracle_out(d, i, t, peers_np, pdt, R_np, rdt)
    e = rel_err(from_dev(out), ref)
    log(f"fused ffn+reduce M={M} h={h} f={f} t={t} i={i} peers={pdt} R={rdt} out={odt}: "
        f"err {e:.4f}")
    assert e <= TOL_BF16


def test_fused_fp32_inputs(gpu):
    M, h, f, t, i = 77, 100, 2 * 52, 2, 1
    d = syn.make_ffn_inputs(710, M, h, f, syn.F32, residual=True)
    X, W1_i, W2_i = dev_inputs(d, i, t)
    peers_np = peers_random(711, t, M, h, syn.F32)
    peers = [None if j == i else to_dev(peers_np[j], syn.F32) for j in range(t)]
    R = to_dev(d["R"], syn.F32)
    out = empty((M, h), syn.F32)
    gpu.tp_ffn_shard_reduce(X, W1_i, W2_i, peers, R, out, i)
    torch.cuda.synchronize()
    ref = oracle_out(d, i, t, peers_np, syn.F32, d["R"], syn.F32)
    e = rel_err(from_dev(out), ref)
    log(f"fused ffn+reduce fp32 inputs: err {e:.3e}")
    assert e <= TOL_F32


@pytest.mark.parametrize("M,h,f,t,i,pdt", [(300, 200, 3 * 424, 3, 2, syn.F32),
                                            (4096, 4096, 16384, 8, 3, syn.BF16),
                                            (2000, 3000, 2 * 2936, 2, 1, syn.BF16)])
def test_fused_equals_unfused_bitwise(gpu, M, h, f, t, i, pdt):
    """The fused call and the same sums done by the unfused calls (the other
    partials + R first, then + Y_i in fp32) agree bit for bit."""
    d = syn.make_ffn_inputs(720 + t, M, h, f, syn.BF16)
    X, W1_i, W2_i = dev_inputs(d, i, t)
    peers = [to_dev(p, pdt) for p in peers_random(721, t, M, h, pdt)]
    R = to_dev(syn.normal_tensor(722, 0, (M, h), 1.0, syn.BF16), syn.BF16)
    fused = empty((M, h), syn.F32)
    gpu.tp_ffn_shard_reduce(X, W1_i, W2_i, [None if j == i else p for j, p in enumerate(peers)],
                            R, fused, i)
    S = empty((M, h), syn.F32)
    gpu.tp_partial_reduce([p for j, p in enumerate(peers) if j != i], R, S)
    Yi = empty((M, h), syn.F32)
    gpu.tp_ffn_shard(X, W1_i, W2_i, Yi, i, t)
    unfused = empty((M, h), syn.F32)
    gpu.tp_partial_reduce([S, Yi], None, unfused)
    torch.cuda.synchronize()
    assert torch.equal(fused, unfused)


def test_fused_repeated_calls_keep_the_stream_order(gpu):
    """Back-to-back fused calls reusing one output and one workspace, with
    inputs changed in between on the caller's stream: every call must see
    its own inputs (the side stream waits for the caller's stream)."""
    M, h, f, t, i = 512, 512, 2048, 4, 1
    d = syn.make_ffn_inputs(740, M, h, f, syn.BF16)
    X, W1_i, W2_i = dev_inputs(d, i, t)
    peers = [None if j == i else to_dev(p, syn.BF16)
             for j, p in enumerate(peers_random(741, t, M, h, syn.BF16))]
    ws = torch.empty(gpu.tp_ffn_shard_reduce_workspace_bytes(M, h, f, t, gpu.TP_BF16),
                     dtype=torch.uint8, device="cuda")
    out = empty((M, h), syn.F32)
    outs, p0s = [], []
    for k in range(3):
        peers[0].mul_(2.0)                   # exact in bf16; on the caller's stream
        p0s.append(peers[0].clone())
        gpu.tp_ffn_shard_reduce(X, W1_i, W2_i, peers, None, out, i, workspace=ws)
        outs.append(out.clone())
    torch.cuda.synchronize()
    Yi = empty((M, h), syn.F32)
    gpu.tp_ffn_shard(X, W1_i, W2_i, Yi, i, t)
    for k in range(3):
        S = empty((M, h), syn.F32)
        gpu.tp_partial_reduce([p0s[k]] + [p for j, p in enumerate(peers) if j not in (0, i)],
                              None, S)
        want = empty((M, h), syn.F32)
        gpu.tp_partial_reduce([S, Yi], None, want)
        torch.cuda.synchronize()
        assert torch.equal(outs[k], want), k


def test_fused_bench_shape_sampled_rows(gpu):
    """t=8, i=3, hidden 4096, 4096 tokens: the other seven shards' bf16
    partials come from tp_ffn_shard, the residual is bf16, out fp32; 128
    sampled rows against the oracle's unsharded FFN + R on those rows."""
    M, h, f, t, i = 4096, 4096, 16384, 8, 3
    d = syn.make_ffn_inputs(2, M, h, f, syn.BF16, residual=True)
    X = to_dev(d["X"], syn.BF16)
    W1 = to_dev(d["W1"], syn.BF16)
    W2 = to_dev(d["W2"], syn.BF16)
    fs = f // t
    peers = []
    for j in range(t):
        if j == i:
            peers.append(None)
            continue
        Y = empty((M, h), syn.BF16)
        gpu.tp_ffn_shard(X, W1[:, j * fs:(j + 1) * fs], W2[j * fs:(j + 1) * fs], Y, j, t)
        peers.append(Y)
    R = to_dev(d["R"], syn.BF16)
    out = empty((M, h), syn.F32)
    gpu.tp_ffn_shard_reduce(X, W1[:, i * fs:(i + 1) * fs], W2[i * fs:(i + 1) * fs], peers, R,
                            out, i)
    torch.cuda.synchronize()
    rows = syn.sample_rows(5, M, 128)
    f64 = {k: syn.to_f64(d[k], syn.BF16) for k in ("X", "W1", "W2", "R")}
    ref = oracle.ffn_full(f64["X"][rows], f64["W1"], f64["W2"]) + f64["R"][rows]
    e = rel_err(from_dev(out)[rows], ref)
    log(f"fused ffn+reduce bench shape, 128 rows: err {e:.4f}")
    assert e <= TOL_BF16


def test_fused_out_may_be_the_residual(gpu):
    M, h, f, t, i = 192, 256, 2 * 256, 2, 0
    d = syn.make_ffn_inputs(730, M, h, f, syn.BF16)
    X, W1_i, W2_i = dev_inputs(d, i, t)
    peers = [None, to_dev(syn.normal_tensor(731, 0, (M, h), 1.0, syn.F32), syn.F32)]
    R = to_dev(syn.normal_tensor(732, 0, (M, h), 1.0, syn.F32), syn.F32)
    ref = empty((M, h), syn.F32)
    gpu.tp_ffn_shard_reduce(X, W1_i, W2_i, peers, R, ref, i)
    gpu.tp_ffn_shard_reduce(X, W1_i, W2_i, peers, R, R, i)      # in place
    torch.cuda.synchronize()
    assert torch.equal(R, ref)
