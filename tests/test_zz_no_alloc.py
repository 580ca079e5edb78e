"""tp_ffn_shard_noalloc (the FFN shard without a workspace, for callers that
cannot allocate) against tp_ffn_shard, through the C ABI: the same kernels,
so the outputs must agree bit for bit.  Calls in a row, each with a smaller
input than the one before (the array keeps the previous call's contents),
then a shape whose GeLU(Z_i) does not fit the array, which must be
rejected."""
import numpy as np
import pytest
import torch

from attention_shards_amd import synthetic as syn
from parity import empty, from_dev, log, to_dev

pytestmark = pytest.mark.gpu


def _inputs(seed, M, h, f, i, t, dtype):
    d = syn.make_ffn_inputs(seed, M, h, f, dtype)
    cols = syn.column_slice(f, i, t)
    X = to_dev(d["X"], dtype)
    W1 = to_dev(d["W1"], dtype)
    W2_i = to_dev(np.ascontiguousarray(d["W2"][cols, :]), dtype)
    return X, W1[:, cols], W2_i


@pytest.mark.parametrize("dtype,out", [(syn.BF16, syn.BF16), (syn.F32, syn.F32)])
def test_noalloc_matches_workspace_entry_point(gpu, dtype, out):
    # the first shape's second product splits K (its fp32 partials sit in the
    # array behind GeLU(Z_i))
    shapes = [(1000, 1000, 8200, 0, 1, 15), (4096, 1024, 8192, 3, 8, 11),
              (300, 200, 3 * 424, 1, 3, 12)]
    if dtype == syn.F32:
        shapes = [(1000, 512, 4 * 512, 2, 4, 13), (77, 100, 2 * 52, 1, 2, 14)]
    for M, h, f, i, t, seed in shapes:
        X, W1_i, W2_i = _inputs(seed, M, h, f, i, t, dtype)
        ref = empty((M, h), out)
        gpu.tp_ffn_shard(X, W1_i, W2_i, ref, i, t)
        got = empty((M, h), out)
        gpu.tp_ffn_shard_noalloc(X, W1_i, W2_i, got, i, t)
        torch.cuda.synchronize()
        a, b = from_dev(got), from_dev(ref)
        log(f"noalloc {dtype} M={M} h={h} f={f} t={t} i={i}: "
            f"max |noalloc - tp_ffn_shard| = {np.max(np.abs(a - b)):.3g}")
        assert np.array_equal(a, b)


def test_noalloc_rejects_shapes_above_its_array(gpu):
    # GeLU(Z_i) of 8192 tokens x 8192 bf16 columns = 128 MiB > 64 MiB
    X = torch.zeros((8192, 64), dtype=torch.bfloat16, device="cuda")
    W1 = torch.zeros((64, 8192), dtype=torch.bfloat16, device="cuda")
    W2 = torch.zeros((8192, 64), dtype=torch.bfloat16, device="cuda")
    Y = torch.empty((8192, 64), dtype=torch.float32, device="cuda")
    assert gpu.tp_ffn_shard_workspace_bytes(8192, 64, 8192, 1, gpu.TP_BF16) > \
        gpu.TP_FFN_NOALLOC_MAX_WORKSPACE
    with pytest.raises(gpu.TPError, match="TP_ERR_WORKSPACE"):
        gpu.tp_ffn_shard_noalloc(X, W1, W2, Y, 0, 1)
