"""Plain fp64 CPU oracle for one GPU's share of a tensor-parallel sub-layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this package; only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` do.  It shares no code with the HIP path
(``attention_shards_amd``): inputs reach it as numpy arrays, already widened
to float64 by the caller.

What it follows: the page "Tensor Parallelism > Combining Column and Row
Parallelism" (mbrenndoerfer.com), i.e. the FFN steps 1-3 (column-parallel
W1 with a local GeLU, row-parallel W2 giving a partial sum, all-reduce), the
multi-head attention decomposition (QKV split by heads, per-head attention,
row-parallel output projection), the residual added after each reduce, and
the layer that chains the two sub-layers, and the sequence-parallel
variant of the sum for the operations the page says are not split across
GPUs (LayerNorm over a row's features): the rows are split instead.

The method reaches the plain unsharded result exactly (up to rounding
order), so every function here is that plain definition written out in
float64, with numpy's matmul as the only library step.  No intermediate is
rounded to a lower precision.

Readings of what the page leaves open (they are listed with reasons in the
design notes at the repository root):
  * GeLU is the exact erf form 0.5*z*(1+erf(z/sqrt 2)); no biases;
  * shard i holds the contiguous block [i*f/t, (i+1)*f/t) of W1's columns
    and W2's rows, and heads [i*n_h/t, (i+1)*n_h/t);
  * attention scores are scaled by 1/sqrt(d), keys j <= query s are kept
    (causal, diagonal included) and the rest are excluded from the softmax;
  * the residual is added once, after the sum of the partials.

Pins: every function is checked, in tests/test_oracle_pins.py, against
invariants the page states (shard-sum identity, local GeLU = slice of the
global GeLU, head independence), closed forms (normal CDF values,
identity weights, prefix means) and brute force on tiny shapes.
"""
from .ffn import gelu, column_parallel, row_parallel, ffn_shard, ffn_full  # noqa: F401
from .attention import attention_heads, attn_shard, attn_full  # noqa: F401
from .reduce import partial_reduce  # noqa: F401
from .layer import layer  # noqa: F401
from .sequence import layernorm, reduce_layernorm  # noqa: F401
