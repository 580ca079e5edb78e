/*
 * tp_shard.h -- C ABI of libtpshard.so: one GPU's share of a Megatron-style
 * tensor-parallel transformer sub-layer, on AMD Instinct MI355X (gfx950).
 *
 * The operations follow the page "Tensor Parallelism > Combining Column and
 * Row Parallelism" (mbrenndoerfer.com):
 *   - FFN, steps 1-2: GPU i receives the full input X, computes
 *     Z_i = X W_{1,i} with its column shard of W1, applies GeLU locally, and
 *     multiplies by its row shard W_{2,i}, which gives a partial sum Y_i over
 *     the full output space                                 -> tp_ffn_shard
 *   - attention: QKV projections split by heads (each GPU holds the Q, K, V
 *     weights of its heads), per-head attention, and the row-parallel output
 *     projection, again a partial sum                       -> tp_attn_shard
 *   - FFN step 3 and the closing paragraph: the partials are summed and the
 *     residual is added to the sum                          -> tp_partial_reduce
 *     (here an in-HBM sum of t buffers on one GPU, not a collective).
 *
 * Conventions shared by every entry point
 *   - Pointers to tensors are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or copies them, and keeps no reference after the
 *     call returns.  They must be 16-byte aligned (TP_ERR_ALIGNMENT).
 *   - Matrices are dense row-major ("X W" orientation: X[M,h], W1[h,f],
 *     W2[f,h]); only W1_i may be a strided view (ld_w1).
 *   - bf16 is bfloat16 (1-8-7), fp32 is IEEE binary32.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *     TP_SUCCESS means "work enqueued on stream": results are stream-ordered
 *     and the caller synchronizes.
 *   - All arguments are validated BEFORE any HIP call; on failure nothing is
 *     enqueued, the status code is returned and tp_last_error_message()
 *     gives a thread-local description.  No C++ exception crosses the ABI.
 *   - Results are bitwise reproducible for the same inputs, shapes and
 *     device: no atomics, fixed summation orders.
 *   - Functions are re-entrant; calls on different streams may run
 *     concurrently as long as their output buffers and workspaces differ.
 */
#ifndef TP_SHARD_H
#define TP_SHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TP_ABI_VERSION 7
#define TP_MAX_PARTIALS 64

/* Element types of tensors crossing the ABI. */
typedef enum {
  TP_F32 = 0,  /* IEEE binary32 */
  TP_BF16 = 1  /* bfloat16, stored as 16-bit words */
} tp_dtype_t;

typedef enum {
  TP_SUCCESS = 0,
  TP_ERR_NULL = 1,          /* a required pointer is NULL */
  TP_ERR_SHAPE = 2,         /* negative size, or size not a multiple of the
                               16-byte vector width along a contiguous dim */
  TP_ERR_SHARD = 3,         /* t < 1, or i outside [0, t) */
  TP_ERR_DIVISIBILITY = 4,  /* ffn % t != 0, or n_heads % t != 0 */
  TP_ERR_DTYPE = 5,         /* unknown dtype code or unsupported combination */
  TP_ERR_WORKSPACE = 6,     /* workspace NULL or smaller than the query says */
  TP_ERR_ALIAS = 7,         /* an output overlaps an input it must not */
  TP_ERR_HIP = 8,           /* a HIP call failed (text in the message) */
  TP_ERR_UNSUPPORTED = 9,   /* valid but not implemented (e.g. head_dim) */
  TP_ERR_ALIGNMENT = 10     /* pointer not 16-byte aligned */
} tp_status_t;

/* ------------------------------------------------------------------------
 * FFN shard (column-parallel W1 + GeLU, then row-parallel W2).
 * ------------------------------------------------------------------------
 * Computes, for this GPU i of t,
 *     Y_i = GeLU(X * W1_i) * W2_i
 * with GeLU(z) = 0.5 z (1 + erf(z / sqrt 2)) (the exact erf form) applied in
 * fp32 to the fp32-accumulated product, and no biases.  Phi(z) is evaluated
 * with the Chebyshev erfc fit of Numerical Recipes (section 6.2, erfcc), so
 * the GeLU value is within 2.5e-7 |z| of the exact one and within a relative
 * 1e-5 of it for every z (also deep in the negative tail).
 *
 *   X     [tokens, hidden]          full input, replicated on every GPU
 *   W1_i  [hidden, ffn/t]           columns [i*ffn/t, (i+1)*ffn/t) of W1;
 *                                   row stride ld_w1 elements: pass 0 or ffn/t
 *                                   for a held shard, ffn for a zero-copy view
 *                                   into a full W1 (pointer W1 + i*ffn/t)
 *   W2_i  [ffn/t, hidden]           rows [i*ffn/t, (i+1)*ffn/t) of W2,
 *                                   contiguous (pointer W2 + i*(ffn/t)*hidden)
 *   Y_i   [tokens, hidden]          output partial, dtype out_dtype
 *   ffn                             the FULL f; this shard has ffn/t columns
 *   in_dtype                        dtype of X, W1_i, W2_i: TP_BF16 (bf16 MFMA,
 *                                   fp32 accumulation, GeLU(Z) rounded to bf16
 *                                   between the GEMMs) or TP_F32 (fp32 MFMA,
 *                                   GeLU(Z) kept in fp32)
 *   out_dtype                       TP_BF16 or TP_F32 (rounded once, nearest-even)
 *   workspace                       device scratch of at least
 *                                   tp_ffn_shard_workspace_bytes(...) bytes; it
 *                                   holds GeLU(Z_i) [tokens, ffn/t] between the
 *                                   two GEMMs (no gather: step 2 reads it as is),
 *                                   bf16 in an internal K-blocked layout
 *                                   (tokens x ffn/t rounded up to 64 columns),
 *                                   fp32 row-major; with bf16 inputs and
 *                                   ffn/t >= 20480 also a K-blocked copy of X
 *                                   (tokens x hidden rounded up to 64 columns)
 *                                   that the first GEMM reads, and, when the
 *                                   second GEMM's tile plan splits its K
 *                                   (ffn/t) into parts, their fp32 partial
 *                                   products (parts x tokens x the split
 *                                   columns); contents are not part of the
 *                                   interface.  The size depends on the
 *                                   current device's compute-unit count (the
 *                                   tile plans do)
 * Shape rules: tokens >= 0 (0 enqueues nothing); hidden and ffn/t multiples
 * of 8 (bf16) or 4 (fp32); ld_w1 >= ffn/t and a multiple of the same; every
 * dimension below 2^31 and tokens*hidden, hidden*ld_w1, tokens*(ffn/t) at
 * most 2^60; with bf16 inputs also hidden, ffn/t < 2^22 and ld_w1 < 2^24
 * (row strides the GEMM tiles address with 32-bit offsets).  The size query
 * returns 0 for an unknown dtype, t < 1 or not dividing ffn, a negative
 * dimension, or one beyond these products and 2^31 limits.
 * Y_i must not overlap X, W1_i, W2_i or the workspace (TP_ERR_ALIAS).
 * The shard index i only selects which pointers the caller passes; it is
 * validated and reported in error messages.
 */
size_t tp_ffn_shard_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn,
                                    int32_t t, int32_t in_dtype);

tp_status_t tp_ffn_shard(const void* X, const void* W1_i, const void* W2_i,
                         void* Y_i, int64_t tokens, int64_t hidden, int64_t ffn,
                         int32_t i, int32_t t, int64_t ld_w1, int32_t in_dtype,
                         int32_t out_dtype, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * FFN shard without allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).
 * ------------------------------------------------------------------------
 * The same computation and kernels as tp_ffn_shard (bit-identical results),
 * with no workspace argument: GeLU(Z_i) lives in a file-scope device array
 * of TP_FFN_NOALLOC_MAX_WORKSPACE bytes inside the library, one per GPU,
 * held from the library's first use on that GPU until the process ends.
 * The call allocates nothing (no hipMalloc, no allocating library routine).
 *   - Shapes whose tp_ffn_shard_workspace_bytes(...) exceeds
 *     TP_FFN_NOALLOC_MAX_WORKSPACE are rejected with TP_ERR_WORKSPACE.
 *   - Every other rule and status is tp_ffn_shard's; the first call on a
 *     device also looks up the array's device address (a failure there is
 *     TP_ERR_HIP).  A rejected call enqueues nothing.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (nothing in it needs to start at zero: GeLU(Z_i) and
 *     any partial products of a split K are written in full before they
 *     are read).  Calls that overlap in time on one GPU (different streams
 *     or host threads without ordering) race on it: order them on one
 *     stream.
 */
#define TP_FFN_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)

tp_status_t tp_ffn_shard_noalloc(const void* X, const void* W1_i, const void* W2_i,
                                 void* Y_i, int64_t tokens, int64_t hidden, int64_t ffn,
                                 int32_t i, int32_t t, int64_t ld_w1, int32_t in_dtype,
                                 int32_t out_dtype, void* stream);

/* ------------------------------------------------------------------------
 * Attention shard (QKV column-parallel by heads, per-head attention,
 * row-parallel output projection).
 * ------------------------------------------------------------------------
 * With nl = n_heads/t local heads of dimension d = head_dim:
 *     [Q | K | V] = X * Wqkv_i
 *     O_h = softmax(Q_h K_h^T / sqrt(d), keys j <= query s if causal) V_h
 *     Y_i = [O_0 | ... | O_{nl-1}] * Wo_i
 * Attention runs within each of the `batch` sequences of length `seq`.
 *
 *   X       [batch*seq, hidden]     bf16, full input
 *   Wqkv_i  [hidden, 3*nl*d]        bf16, columns laid out [W_Q,i | W_K,i |
 *                                   W_V,i], each head-major (local head j in
 *                                   columns j*d .. j*d+d-1 of its block); the
 *                                   heads are [i*nl, (i+1)*nl) of the model
 *   Wo_i    [nl*d, hidden]          bf16, rows of those heads in W_o
 *   Y_i     [batch*seq, hidden]     output partial, out_dtype TP_F32 or TP_BF16
 *   causal                          1: key j is kept for query s iff j <= s;
 *                                   0: all keys kept
 *   in_dtype                        TP_BF16 only
 * Internals (exposed only through the workspace size): Q and K are kept in
 * fp16 (11 significant bits) and V as an fp16 hi+lo pair (hi = fp16(v),
 * lo = fp16(v - hi)), so the value product carries about 22 significant
 * bits; softmax runs in fp32 with the probabilities rounded to fp16; the
 * head outputs O are kept as fp16 plus their residual in bf8 (e5m2), about
 * 14 significant bits, and the output projection multiplies the fp16 part
 * by Wo_i converted to fp16 and the residual by Wo_i converted to bf8 in one
 * pass over K.  Q, K and V must lie within the fp16 range (|value| <
 * 65504), Wo_i within bf8's (|value| <= 57344); Wo_i entries below 2^-14 in
 * magnitude keep fp16's absolute resolution of 2^-24.  The workspace size
 * depends on the current device's compute-unit count (the attention work
 * split does).
 * Shape rules: batch, seq >= 0; head_dim == 128; hidden multiple of 8;
 * batch, batch*seq and batch*(n_heads/t)*ceil(seq/64) below 2^31; hidden and
 * 2*(n_heads/t)*head_dim below 2^22; seq below 2^23 (32-bit tile offsets in
 * the GEMMs and the attention kernel).  The size query returns 0 for any
 * shape these rules (or n_heads % t, head_dim) reject.
 */
size_t tp_attn_shard_workspace_bytes(int64_t batch, int64_t seq, int32_t n_heads,
                                     int32_t head_dim, int32_t t);

tp_status_t tp_attn_shard(const void* X, const void* Wqkv_i, const void* Wo_i,
                          void* Y_i, int64_t batch, int64_t seq, int64_t hidden,
                          int32_t n_heads, int32_t head_dim, int32_t i,
                          int32_t t, int32_t causal, int32_t in_dtype,
                          int32_t out_dtype, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Sum of the t partials plus the residual (one-GPU stand-in for the
 * all-reduce of FFN step 3, followed by the residual add).
 * ------------------------------------------------------------------------
 *     out = (partials[0] + partials[1] + ... + partials[t-1]) + residual
 * accumulated in fp32 in that fixed order (i ascending, residual last) and
 * rounded once to out_dtype.
 *
 *   partials   HOST array of t device pointers, each [rows, cols] of
 *              partial_dtype; 1 <= t <= TP_MAX_PARTIALS
 *   residual   device [rows, cols] of residual_dtype, or NULL for none
 *   out        device [rows, cols] of out_dtype; it MAY be the same buffer as
 *              residual or partials[0] when the dtypes match (each element is
 *              read before it is written); any other overlap is TP_ERR_ALIAS
 * Shape rules: rows, cols >= 0; cols a multiple of 8; rows*cols <= 2^60.
 */
tp_status_t tp_partial_reduce(const void* const* partials, int32_t t,
                              const void* residual, void* out, int64_t rows,
                              int64_t cols, int32_t partial_dtype,
                              int32_t residual_dtype, int32_t out_dtype,
                              void* stream);

/* ------------------------------------------------------------------------
 * One row block of that sum: the reduce-scatter half of the all-reduce
 * (each of nslices GPUs reduces its own row block of all t partials, read
 * in place, before an all-gather of the blocks; page "Tensor Parallelism >
 * Combining Column and Row Parallelism", FFN step 3).
 * ------------------------------------------------------------------------
 * The pointers and rows, cols describe the full [rows, cols] tensors, as for
 * tp_partial_reduce.  Only rows [r0, r1) of out are written, with
 *     r0 = slice * (rows / nslices) + min(slice, rows % nslices),
 *     r1 = r0 + rows / nslices + (slice < rows % nslices ? 1 : 0),
 * so the nslices blocks tile [0, rows) and differ by at most one row; each
 * element is computed exactly as tp_partial_reduce computes it (the same
 * order and rounding), so the blocks of all slices together equal the full
 * reduce bit for bit.  The partial pointers may belong to other devices
 * (peer-mapped memory); nothing else is read or written.
 *   slice, nslices  0 <= slice < nslices (TP_ERR_SHARD otherwise)
 * Other arguments, aliasing and shape rules: those of tp_partial_reduce,
 * applied to the block.  An empty block (rows < nslices) enqueues nothing.
 */
tp_status_t tp_partial_reduce_slice(const void* const* partials, int32_t t,
                                    const void* residual, void* out, int64_t rows,
                                    int64_t cols, int32_t slice, int32_t nslices,
                                    int32_t partial_dtype, int32_t residual_dtype,
                                    int32_t out_dtype, void* stream);

/* ------------------------------------------------------------------------
 * Sequence-parallel sum + LayerNorm (the operations the page "Combining
 * Column and Row Parallelism" names as reductions over the whole feature
 * dimension, which are not split across GPUs by columns; the rows are split
 * instead).
 * ------------------------------------------------------------------------
 * For the rows [r0, r1) of block `slice` of `nslices` (balanced blocks as in
 * tp_partial_reduce_slice), with all rows full width:
 *     x = (partials[0] + ... + partials[t-1]) + residual      (as the reduce)
 *     y = (x - mean(x)) / sqrt(var(x) + eps) * gamma + beta   (per row)
 * mean and the biased variance over the row's `cols` features, in fp32;
 * that is the reduce-scatter half of the all-reduce, LayerNorm on this GPU's
 * rows, and -- since block j writes rows [r0, r1) of x_out and ln_out in
 * place -- the all-gather half when the blocks of all slices land in the
 * same buffers.
 *
 *   partials   HOST array of t device pointers, each [rows, cols] of
 *              partial_dtype (the whole matrices; only the block is read)
 *   residual   [rows, cols] of residual_dtype, or NULL
 *   x_out      [rows, cols] of x_dtype, or NULL (x not stored); may be
 *              exactly one of the inputs of the same element size
 *   ln_out     [rows, cols] of ln_dtype; overlaps nothing else
 *   gamma,beta fp32 [cols] device arrays, or NULL (1 and 0)
 *   eps        added to the variance inside the square root, >= 0
 * Shape rules: cols a multiple of 8 and at most 32768 (one row stays in the
 * registers of a workgroup); rows * cols at most 2^60.
 */
tp_status_t tp_sp_reduce_layernorm(const void* const* partials, int32_t t, const void* residual,
                                   void* x_out, void* ln_out, const float* gamma,
                                   const float* beta, float eps, int64_t rows, int64_t cols,
                                   int32_t slice, int32_t nslices, int32_t partial_dtype,
                                   int32_t residual_dtype, int32_t x_dtype, int32_t ln_dtype,
                                   void* stream);

/* ------------------------------------------------------------------------
 * FFN shard fused with the sum of the partials and the residual: the
 * one-GPU counterpart of overlapping the row-parallel product with the
 * all-reduce (the page's note on hiding communication behind the GEMMs).
 * ------------------------------------------------------------------------
 *     out = ((sum over j != i, in j order, of P_j) + residual) + P_i
 * where P_i = GeLU(X * W1_i) * W2_i is computed as tp_ffn_shard computes
 * Y_i but added from its fp32 accumulators (never rounded or stored), and
 * P_j (j != i) are the other shards' partials, read from peer_partials[j].
 * Accumulation is fp32 in the order written; out is rounded once to
 * out_dtype.  The sum of the other operands runs on a second stream of the
 * library (one per device, created on first use and kept until the process
 * ends) concurrently with the first GEMM; the second GEMM's epilogue adds
 * it, so neither Y_i nor a separate pass over all t partials goes through
 * memory after the product.  Calls from several host threads are
 * serialized while they enqueue.
 *
 *   X, W1_i, W2_i, tokens, hidden, ffn, i, t, ld_w1, in_dtype:
 *                  as for tp_ffn_shard
 *   peer_partials  HOST array of t device pointers, each [tokens, hidden] of
 *                  partial_dtype; entry i is not read (may be NULL);
 *                  1 <= t <= TP_MAX_PARTIALS (may be NULL when t == 1)
 *   residual       device [tokens, hidden] of residual_dtype, or NULL
 *   out            device [tokens, hidden] of out_dtype; it MAY be the same
 *                  buffer as the residual or a peer partial when the element
 *                  sizes match; any other overlap with an input, a peer
 *                  partial, the residual or the workspace is TP_ERR_ALIAS,
 *                  and so is a workspace that overlaps a peer partial or the
 *                  residual
 *   workspace      at least tp_ffn_shard_reduce_workspace_bytes(...) bytes:
 *                  GeLU(Z_i) as for tp_ffn_shard, then the fp32 sum of the
 *                  other operands [tokens, hidden]
 * Shape rules: those of tp_ffn_shard.
 */
size_t tp_ffn_shard_reduce_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn,
                                           int32_t t, int32_t in_dtype);

tp_status_t tp_ffn_shard_reduce(const void* X, const void* W1_i, const void* W2_i,
                                const void* const* peer_partials,
                                const void* residual, void* out, int64_t tokens,
                                int64_t hidden, int64_t ffn, int32_t i, int32_t t,
                                int64_t ld_w1, int32_t in_dtype,
                                int32_t partial_dtype, int32_t residual_dtype,
                                int32_t out_dtype, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Static text for a status code ("TP_SUCCESS", ...). Never NULL. */
const char* tp_status_string(int32_t status);

/* Thread-local detail of the last non-success return on this thread ("" if
 * none).  Valid until the next call into the library on the same thread. */
const char* tp_last_error_message(void);

/* TP_ABI_VERSION of the built library. */
int32_t tp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TP_SHARD_H */
