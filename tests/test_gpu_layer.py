"""A whole transformer layer with t shards on one GPU (attention sub-layer,
sum + residual, FFN sub-layer, sum + residual) through the C ABI, against
the fp64 unsharded layer of the oracle."""
import numpy as np
import pytest
import torch

import oracle
from attention_shards_amd import layer as L
from attention_shards_amd import synthetic as syn
from parity import TOL_BF16, bf16_floor, from_dev, log, rel_err, to_dev

pytestmark = pytest.mark.gpu


def run_layer(a, batch, seq, nh, d, f, t, ffn_partial_dtype=torch.float32):
    X = to_dev(a["X"], syn.BF16)
    Wqkv = [to_dev(syn.qkv_held_shard(a["WQ"], a["WK"], a["WV"], nh, d, i, t), syn.BF16)
            for i in range(t)]
    Wo = [to_dev(np.ascontiguousarray(a["WO"][syn.head_slice(nh, d, i, t), :]), syn.BF16)
          for i in range(t)]
    W1 = to_dev(a["W1"], syn.BF16)
    W2 = to_dev(a["W2"], syn.BF16)
    fs = f // t
    X1, X2 = L.layer_forward(X, Wqkv, Wo, [W1[:, i * fs:(i + 1) * fs] for i in range(t)],
                             [W2[i * fs:(i + 1) * fs] for i in range(t)], batch, seq, nh, d,
                             True, ffn_partial_dtype)
    torch.cuda.synchronize()
    return from_dev(X1), from_dev(X2)


def ref_layer(a, batch, seq, nh, d):
    f = {k: syn.to_f64(a[k], syn.BF16) for k in ("X", "WQ", "WK", "WV", "WO", "W1", "W2")}
    return oracle.layer(f["X"], f["WQ"], f["WK"], f["WV"], f["WO"], f["W1"], f["W2"],
                        batch, seq, nh, d)


@pytest.mark.parametrize("batch,seq,h,nh,f,t,pdt", [
    (2, 96, 256, 4, 1024, 2, torch.float32),     # ragged sequences, two shards
    (1, 130, 512, 4, 2048, 4, torch.bfloat16),   # bf16 FFN partials, four shards
    (1, 1024, 2048, 16, 8192, 4, torch.float32),
])
def test_layer_matches_unsharded_fp64(gpu, batch, seq, h, nh, f, t, pdt):
    d = 128
    a = syn.make_layer_inputs(500 + seq, batch, seq, h, nh, d, f)
    X1, X2 = run_layer(a, batch, seq, nh, d, f, t, pdt)
    R1, R2 = ref_layer(a, batch, seq, nh, d)
    e1, e2 = rel_err(X1, R1), rel_err(X2, R2)
    log(f"layer batch={batch} seq={seq} h={h} heads={nh} f={f} t={t} ffn partials={pdt}: "
        f"X1 err {e1:.4f}, X2 err {e2:.4f} (bf16 floors {bf16_floor(R1):.4f}, "
        f"{bf16_floor(R2):.4f})")
    assert e1 <= TOL_BF16 and e2 <= TOL_BF16


def test_layer_shard_count_does_not_change_result(gpu):
    """t=1 and t=4 give the same layer up to fp32 reassociation and the
    bf16 rounding of Z (which depends only on the element, not the shard)."""
    batch, seq, h, nh, f, d = 1, 200, 512, 4, 2048, 128
    a = syn.make_layer_inputs(601, batch, seq, h, nh, d, f)
    _, Y1 = run_layer(a, batch, seq, nh, d, f, 1)
    _, Y4 = run_layer(a, batch, seq, nh, d, f, 4)
    e = rel_err(Y4, Y1)
    log(f"layer t=4 vs t=1 on the GPU: {e:.2e}")
    assert e <= 1e-4
