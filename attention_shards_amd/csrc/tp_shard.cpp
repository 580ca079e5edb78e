// C ABI of libtpshard.so: argument validation, workspace layout and launch
// sequencing for one GPU's share of a tensor-parallel transformer sub-layer
// (page "Tensor Parallelism > Combining Column and Row Parallelism").
//
// Every check runs before the first kernel launch, so a rejected call
// enqueues nothing and changes no device state; besides the launches
// (through the tp:: launchers) and error queries, the only HIP calls are
// reads of the current device and its compute-unit count, which the
// attention work split (and so its workspace size) depends on.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/tp_shard.h"
#include "internal.h"

namespace {

thread_local std::string g_err;

tp_status_t fail(tp_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

tp_status_t ok() {
  g_err.clear();
  return TP_SUCCESS;
}

bool valid_dtype(int32_t d) { return d == TP_F32 || d == TP_BF16; }
int64_t esize(int32_t d) { return d == TP_F32 ? 4 : 2; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + (uintptr_t)(bytes > 0 ? bytes : 0)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

// Bytes spanned by a [rows, cols] view with row stride ld.
int64_t span_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t es) {
  if (rows <= 0 || cols <= 0) return 0;
  return ((rows - 1) * ld + cols) * es;
}

tp_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kInt32Max = 2147483647;
// Largest element count of one operand: its byte extent (at most 4 bytes an
// element) then stays far inside int64, also for fp32 dimensions, which are
// otherwise bounded only by 2^31 - 1 each.
constexpr int64_t kMaxElems = int64_t(1) << 60;
bool fits(int64_t a, int64_t b) { return a <= 0 || b <= kMaxElems / a; }
// The bf16 GEMMs address a tile through a buffer descriptor with 32-bit byte
// offsets: up to 256 rows of A (row stride lda) and 64 rows of B (ldb) per
// tile, so lda < 2^22 and ldb < 2^24 elements.  The attention kernel reads
// 128 V^T rows of seq_pad keys the same way, so seq_pad < 2^23.
constexpr int64_t kMaxLdA = int64_t(1) << 22;
constexpr int64_t kMaxLdB = int64_t(1) << 24;
constexpr int64_t kMaxSeqPad = int64_t(1) << 23;
// bf16 FFN workspace: GeLU(Z_i) is kept K-blocked, [ceil(F/kb)][tokens][kb]
// with kb = 32 or 64 (the second product's stage depth), so its column count
// is rounded up to a multiple of 64.
constexpr int64_t kZBlock = 64;
// For shards of at least this many ffn columns GEMM1 reads X K-blocked too
// (a copy of X in the workspace, [ceil(h/kb)][tokens][kb]): every stage's A
// tile is then one contiguous run instead of 128-byte pieces of 256 rows.
// The copy moves 4 tokens h bytes, the main loop gains 2-3% over reading X
// row-major (same-box first products: 6302 vs 6520 us at 2048 x 22528 x
// 90112, 422 vs 431 us at 2048 x 16384 x 8192, 1898 vs 1904 us at 8192 x
// 12288 x 12288; the copies 30, 23, 60 us), which pays for the copy from
// about 20 000 columns on.
constexpr int64_t kXBlockMinCols = 20480;

// Bytes of the K-blocked copy of X (0 when GEMM1 reads X as given).
int64_t x_kblock_bytes(int64_t tokens, int64_t hidden, int64_t fs, int32_t in_dtype) {
  if (in_dtype != TP_BF16 || fs < kXBlockMinCols) return 0;
  return (tokens * ((hidden + kZBlock - 1) / kZBlock * kZBlock) * 2 + 255) / 256 * 256;
}

// Bytes of the fp32 partials of GEMM2 when its plan splits K (bf16 inputs;
// the dimensions have passed the ABI checks).
int64_t split_partial_bytes(int64_t tokens, int64_t hidden, int64_t fs, int32_t in_dtype) {
  if (in_dtype != TP_BF16 || tokens <= 0 || tokens > 2147483647 || hidden > 2147483647)
    return 0;
  return (tp::gemm_bf16_split_bytes((int)tokens, (int)hidden, fs) + 255) / 256 * 256;
}
constexpr int64_t kAttnHeadDim = 128;
constexpr int64_t kAttnKeyTile = 64;

int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

// The attention shapes the kernels address (checked by tp_attn_shard before
// anything else uses them, and by its workspace query): tokens and the
// (sequence, head, key tile) count within int32, V^T rows of seq_pad keys
// and the [Q | K | V] and O row widths within the 32-bit buffer offsets.
bool attn_shape_ok(int64_t batch, int64_t seq, int64_t nl) {
  if (batch < 0 || seq < 0 || nl < 1 || batch > kInt32Max || nl > kInt32Max) return false;
  if (seq > 0 && batch > kInt32Max / seq) return false;  // tokens
  const int64_t seq_pad = (seq + kAttnKeyTile - 1) / kAttnKeyTile * kAttnKeyTile;
  return 3 * nl * kAttnHeadDim <= kInt32Max && 2 * nl * kAttnHeadDim < kMaxLdA &&
         seq_pad < kMaxSeqPad && batch * nl <= kInt32Max &&
         batch * nl * (seq_pad / kAttnKeyTile) <= kInt32Max;
}

// Attention workspace: four [batch*nl, seq_pad, d] 16-bit arrays (Q, K in
// fp16, V^T as an fp16 hi/lo pair) followed by O [batch*seq, nl*d] as fp16
// plus a bf8 residual (3 bytes per element), then the partial results of
// split query blocks (fp32).
constexpr int64_t kAttnParts = 4;
struct AttnLayout {
  int64_t seq_pad, part_bytes, o_bytes, split_bytes, total;
};
AttnLayout attn_layout(int64_t batch, int64_t seq, int64_t nl, int64_t d) {
  AttnLayout L;
  L.seq_pad = (seq + kAttnKeyTile - 1) / kAttnKeyTile * kAttnKeyTile;
  L.part_bytes = align256(batch * nl * L.seq_pad * d * 2);
  L.o_bytes = align256(batch * seq * nl * d * 3);
  L.split_bytes = align256(tp::attn_partial_bytes((int)batch, (int)seq, (int)nl));
  L.total = kAttnParts * L.part_bytes + L.o_bytes + L.split_bytes;
  return L;
}

}  // namespace

extern "C" {

int32_t tp_abi_version(void) { return TP_ABI_VERSION; }

const char* tp_status_string(int32_t s) {
  switch (s) {
    case TP_SUCCESS: return "TP_SUCCESS";
    case TP_ERR_NULL: return "TP_ERR_NULL";
    case TP_ERR_SHAPE: return "TP_ERR_SHAPE";
    case TP_ERR_SHARD: return "TP_ERR_SHARD";
    case TP_ERR_DIVISIBILITY: return "TP_ERR_DIVISIBILITY";
    case TP_ERR_DTYPE: return "TP_ERR_DTYPE";
    case TP_ERR_WORKSPACE: return "TP_ERR_WORKSPACE";
    case TP_ERR_ALIAS: return "TP_ERR_ALIAS";
    case TP_ERR_HIP: return "TP_ERR_HIP";
    case TP_ERR_UNSUPPORTED: return "TP_ERR_UNSUPPORTED";
    case TP_ERR_ALIGNMENT: return "TP_ERR_ALIGNMENT";
    default: return "TP_ERR_UNKNOWN_STATUS";
  }
}

const char* tp_last_error_message(void) { return g_err.c_str(); }

// ---------------------------------------------------------------------------
// FFN shard
// ---------------------------------------------------------------------------
size_t tp_ffn_shard_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn,
                                    int32_t t, int32_t in_dtype) {
  if (tokens < 0 || hidden < 0 || ffn <= 0 || t < 1 || ffn % t != 0 || !valid_dtype(in_dtype))
    return 0;
  // bf16: GeLU(Z_i) K-blocked in blocks of up to 64 columns (kZBlock), then
  // for wide shards the K-blocked copy of X, then the fp32 partials of GEMM2
  // when its plan splits K
  const int64_t fs = ffn / t;
  const int64_t cols = in_dtype == TP_BF16 ? (fs + kZBlock - 1) / kZBlock * kZBlock : fs;
  // shapes tp_ffn_shard rejects for their size (0, not a wrapped product)
  if (tokens > kInt32Max || hidden > kInt32Max || fs > kInt32Max || !fits(tokens, cols) ||
      !fits(tokens, hidden))
    return 0;
  return (size_t)(align256(tokens * cols * esize(in_dtype)) +
                  x_kblock_bytes(tokens, hidden, fs, in_dtype) +
                  split_partial_bytes(tokens, hidden, fs, in_dtype));
}

}  // extern "C"

namespace {

// Checks shared by tp_ffn_shard and tp_ffn_shard_reduce, in the order the
// ABI documents them.  On success *fs_out = ffn/t and *ld_w1 is resolved.
// `out` / `out_bytes` is the output tensor checked against the inputs.
// With check_ws false the workspace checks (NULL, alignment, size, overlap)
// are skipped: the argument checks of a caller that brings its own memory.
tp_status_t check_ffn(const char* fn, const void* X, const void* W1_i, const void* W2_i,
                      const void* out, int64_t out_bytes, int64_t tokens, int64_t hidden,
                      int64_t ffn, int32_t i, int32_t t, int64_t* ld_w1, int32_t in_dtype,
                      int32_t out_dtype, const void* workspace, size_t workspace_bytes,
                      int64_t* fs_out, bool check_ws = true) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(TP_ERR_DTYPE, "%s: dtype codes in=%d out=%d", fn, in_dtype, out_dtype);
  if (t < 1 || i < 0 || i >= t) return fail(TP_ERR_SHARD, "%s: shard i=%d of t=%d", fn, i, t);
  if (tokens < 0 || hidden <= 0 || ffn <= 0)
    return fail(TP_ERR_SHAPE, "%s(i=%d): tokens=%lld hidden=%lld ffn=%lld", fn, i,
                (long long)tokens, (long long)hidden, (long long)ffn);
  if (ffn % t != 0)
    return fail(TP_ERR_DIVISIBILITY, "%s(i=%d): ffn=%lld not divisible by t=%d", fn, i,
                (long long)ffn, t);
  const int64_t fs = ffn / t;
  const int64_t es = esize(in_dtype);
  const int64_t vec = 16 / es;
  if (*ld_w1 == 0) *ld_w1 = fs;
  if (hidden % vec || fs % vec || *ld_w1 % vec || *ld_w1 < fs)
    return fail(TP_ERR_SHAPE,
                "%s(i=%d): hidden=%lld, ffn/t=%lld and ld_w1=%lld must be multiples "
                "of %lld with ld_w1 >= ffn/t",
                fn, i, (long long)hidden, (long long)fs, (long long)*ld_w1, (long long)vec);
  if (tokens > kInt32Max || hidden > kInt32Max || fs > kInt32Max)
    return fail(TP_ERR_SHAPE, "%s(i=%d): a dimension exceeds 2^31-1", fn, i);
  if (!fits(tokens, hidden) || !fits(hidden, *ld_w1) || !fits(tokens, fs))
    return fail(TP_ERR_SHAPE, "%s(i=%d): an operand exceeds 2^60 elements", fn, i);
  if (in_dtype == TP_BF16 && (hidden >= kMaxLdA || fs >= kMaxLdA || *ld_w1 >= kMaxLdB))
    return fail(TP_ERR_SHAPE,
                "%s(i=%d): bf16 needs hidden and ffn/t below 2^22 and ld_w1 below 2^24 "
                "(hidden=%lld ffn/t=%lld ld_w1=%lld)",
                fn, i, (long long)hidden, (long long)fs, (long long)*ld_w1);
  *fs_out = fs;
  if (tokens == 0) return ok();
  if (!X || !W1_i || !W2_i || !out)
    return fail(TP_ERR_NULL, "%s(i=%d): NULL tensor pointer", fn, i);
  if (check_ws && !workspace) return fail(TP_ERR_WORKSPACE, "%s(i=%d): NULL workspace", fn, i);
  if (!aligned16(X) || !aligned16(W1_i) || !aligned16(W2_i) || !aligned16(out) ||
      (check_ws && !aligned16(workspace)))
    return fail(TP_ERR_ALIGNMENT, "%s(i=%d): pointers must be 16-byte aligned", fn, i);
  const size_t need = tp_ffn_shard_workspace_bytes(tokens, hidden, ffn, t, in_dtype);
  if (check_ws && workspace_bytes < need)
    return fail(TP_ERR_WORKSPACE, "%s(i=%d): workspace %zu bytes < %zu needed", fn, i,
                workspace_bytes, need);
  const Range rx = range_of(X, tokens * hidden * es);
  const Range rw1 = range_of(W1_i, span_bytes(hidden, fs, *ld_w1, es));
  const Range rw2 = range_of(W2_i, fs * hidden * es);
  const Range ry = range_of(out, out_bytes);
  if (!check_ws) {
    if (overlap(ry, rx) || overlap(ry, rw1) || overlap(ry, rw2))
      return fail(TP_ERR_ALIAS, "%s(i=%d): the output overlaps an input", fn, i);
    return ok();
  }
  // the extent GEMM1 writes: with bf16 inputs GeLU(Z_i) is K-blocked over
  // ffn/t rounded up to 64 columns, which the size query covers
  const Range rws = range_of(workspace, (int64_t)need);
  if (overlap(ry, rx) || overlap(ry, rw1) || overlap(ry, rw2) || overlap(ry, rws))
    return fail(TP_ERR_ALIAS, "%s(i=%d): the output overlaps an input or the workspace", fn, i);
  if (overlap(rws, rx) || overlap(rws, rw1) || overlap(rws, rw2))
    return fail(TP_ERR_ALIAS, "%s(i=%d): workspace overlaps an input", fn, i);
  return ok();
}

}  // namespace

namespace tp {

tp_status_t ffn_check_args(const char* fn, const void* X, const void* W1_i, const void* W2_i,
                           const void* Y_i, int64_t tokens, int64_t hidden, int64_t ffn,
                           int32_t i, int32_t t, int64_t ld_w1, int32_t in_dtype,
                           int32_t out_dtype) {
  try {
    int64_t fs = 0;
    return check_ffn(fn, X, W1_i, W2_i, Y_i,
                     valid_dtype(out_dtype) ? tokens * hidden * esize(out_dtype) : 0, tokens,
                     hidden, ffn, i, t, &ld_w1, in_dtype, out_dtype, nullptr, 0, &fs, false);
  } catch (...) {
    return fail(TP_ERR_HIP, "%s: internal exception", fn);
  }
}

tp_status_t set_error(tp_status_t st, const char* msg) { return fail(st, "%s", msg); }

}  // namespace tp

namespace {

// One side stream and two events per device for the fused FFN + reduce: the
// sum of the other operands runs on the side stream while GEMM1 runs on the
// caller's stream.  Created on first use, at the default priority, kept
// until the process ends; `m` serializes the enqueue sequences of calls from
// several host threads (the events are reused).
struct SideStream {
  std::mutex m;
  bool ready = false;
  hipStream_t s = nullptr;
  hipEvent_t inputs_ready = nullptr, others_summed = nullptr;
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];

hipError_t side_stream(int dev, SideStream** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  SideStream& ss = g_side[dev];
  *out = &ss;
  if (ss.ready) return hipSuccess;
  hipError_t e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.inputs_ready, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.others_summed, hipEventDisableTiming);
  if (e == hipSuccess) ss.ready = true;
  return e;
}

// GEMM2's fp32 partials in the bf16 workspace, behind GeLU(Z_i) and the
// K-blocked copy of X (nullptr when GEMM2's plan does not split K).
float* split_partials(void* workspace, int64_t M, int64_t H, int64_t F, int32_t in_dtype) {
  if (split_partial_bytes(M, H, F, in_dtype) == 0) return nullptr;
  return reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                  align256(M * ((F + kZBlock - 1) / kZBlock * kZBlock) * 2) +
                                  x_kblock_bytes(M, H, F, in_dtype));
}

// GEMM1 + GeLU into the workspace.  bf16: GeLU(Z_i) is stored K-blocked
// in the block depth of the kernel GEMM2 will run (its A tiles are then
// contiguous runs of memory; GEMM2 is planned over its K = F, which may
// split it); fp32: row-major.
hipError_t ffn_gemm1(const void* X, const void* W1_i, int64_t ld_w1, void* workspace, int M,
                     int H, int F, int32_t in_dtype, hipStream_t s) {
  if (in_dtype == TP_BF16 && x_kblock_bytes(M, H, F, in_dtype) > 0) {
    // X copied K-blocked (in GEMM1's stage depth) behind GeLU(Z_i)
    uint16_t* xkb = reinterpret_cast<uint16_t*>(
        static_cast<char*>(workspace) + align256((int64_t)M * ((F + kZBlock - 1) / kZBlock * kZBlock) * 2));
    const int kb1 = tp::gemm_bf16_a_block(M, F, 0);
    hipError_t e = tp::kblock_bf16(static_cast<const uint16_t*>(X), H, xkb, M, H, kb1, s);
    if (e != hipSuccess) return e;
    return tp::gemm_bf16_gelu_akb(xkb, kb1, static_cast<const uint16_t*>(W1_i), ld_w1,
                                  static_cast<uint16_t*>(workspace), M, F, H,
                                  tp::gemm_bf16_a_block(M, H, F), s);
  }
  if (in_dtype == TP_BF16)
    return tp::gemm_bf16_gelu(static_cast<const uint16_t*>(X), H,
                              static_cast<const uint16_t*>(W1_i), ld_w1,
                              static_cast<uint16_t*>(workspace), F, M, F, H,
                              tp::gemm_bf16_a_block(M, H, F), s);
  return tp::gemm_f32(static_cast<const float*>(X), H, static_cast<const float*>(W1_i), ld_w1,
                      workspace, F, tp::OUT_F32, true, M, F, H, s);
}

}  // namespace

extern "C" {

tp_status_t tp_ffn_shard(const void* X, const void* W1_i, const void* W2_i,
                         void* Y_i, int64_t tokens, int64_t hidden, int64_t ffn,
                         int32_t i, int32_t t, int64_t ld_w1, int32_t in_dtype,
                         int32_t out_dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
  try {
    int64_t fs = 0;
    const tp_status_t st =
        check_ffn("tp_ffn_shard", X, W1_i, W2_i, Y_i, tokens * hidden * esize(out_dtype),
                  tokens, hidden, ffn, i, t, &ld_w1, in_dtype, out_dtype, workspace,
                  workspace_bytes, &fs);
    if (st != TP_SUCCESS || tokens == 0) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const int M = (int)tokens, H = (int)hidden, F = (int)fs;
    hipError_t e = ffn_gemm1(X, W1_i, ld_w1, workspace, M, H, F, in_dtype, s);
    if (e != hipSuccess) return hip_status(e, "tp_ffn_shard: GEMM1 launch");
    const tp::OutType ot = out_dtype == TP_F32 ? tp::OUT_F32 : tp::OUT_BF16;
    if (in_dtype == TP_BF16)
      e = tp::gemm_bf16_store_kb(static_cast<const uint16_t*>(workspace),
                                 tp::gemm_bf16_a_block(M, H, F),
                                 static_cast<const uint16_t*>(W2_i), H, Y_i, H, ot, M, H, F,
                                 split_partials(workspace, M, H, F, in_dtype), s);
    else
      e = tp::gemm_f32(static_cast<const float*>(workspace), F,
                       static_cast<const float*>(W2_i), H, Y_i, H, ot, false, M, H, F, s);
    return hip_status(e, "tp_ffn_shard: GEMM2 launch");
  } catch (...) {
    return fail(TP_ERR_HIP, "tp_ffn_shard: internal exception");
  }
}

size_t tp_ffn_shard_reduce_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn,
                                           int32_t t, int32_t in_dtype) {
  const size_t z = tp_ffn_shard_workspace_bytes(tokens, hidden, ffn, t, in_dtype);
  if (z == 0 || hidden <= 0) return 0;
  return z + (size_t)align256(tokens * hidden * 4);
}

tp_status_t tp_ffn_shard_reduce(const void* X, const void* W1_i, const void* W2_i,
                                const void* const* peer_partials,
                                const void* residual, void* out, int64_t tokens,
                                int64_t hidden, int64_t ffn, int32_t i, int32_t t,
                                int64_t ld_w1, int32_t in_dtype,
                                int32_t partial_dtype, int32_t residual_dtype,
                                int32_t out_dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
  const char* fn = "tp_ffn_shard_reduce";
  try {
    if (!valid_dtype(partial_dtype) || (residual && !valid_dtype(residual_dtype)))
      return fail(TP_ERR_DTYPE, "%s: dtype codes partial=%d residual=%d", fn, partial_dtype,
                  residual_dtype);
    if (t > TP_MAX_PARTIALS)
      return fail(TP_ERR_SHARD, "%s: t=%d above %d", fn, t, TP_MAX_PARTIALS);
    int64_t fs = 0;
    const int64_t n = tokens * hidden;
    const int64_t ob = esize(out_dtype);
    // the GEMM checks, with the Z part of the workspace
    tp_status_t st = check_ffn(fn, X, W1_i, W2_i, out, n * ob, tokens, hidden, ffn, i, t,
                               &ld_w1, in_dtype, out_dtype, workspace, workspace_bytes, &fs);
    if (st != TP_SUCCESS || tokens == 0) return st;
    const size_t need = tp_ffn_shard_reduce_workspace_bytes(tokens, hidden, ffn, t, in_dtype);
    if (workspace_bytes < need)
      return fail(TP_ERR_WORKSPACE, "%s(i=%d): workspace %zu bytes < %zu needed", fn, i,
                  workspace_bytes, need);
    if (t > 1 && !peer_partials) return fail(TP_ERR_NULL, "%s(i=%d): NULL peer array", fn, i);
    const size_t z_bytes = tp_ffn_shard_workspace_bytes(tokens, hidden, ffn, t, in_dtype);
    float* S = reinterpret_cast<float*>(static_cast<char*>(workspace) + z_bytes);
    const Range ro = range_of(out, n * ob);
    const Range rws = range_of(workspace, (int64_t)need);
    if (overlap(ro, rws))
      return fail(TP_ERR_ALIAS, "%s(i=%d): out overlaps the workspace", fn, i);
    const int64_t pb = esize(partial_dtype);
    tp::ReducePtrs ptrs;
    int np = 0;  // the other shards' partials, in j order
    for (int k = 0; k < t; ++k) {
      if (k == i) continue;
      const void* p = peer_partials[k];
      if (!p) return fail(TP_ERR_NULL, "%s(i=%d): peer_partials[%d] is NULL", fn, i, k);
      if (!aligned16(p))
        return fail(TP_ERR_ALIGNMENT, "%s(i=%d): peer_partials[%d] not 16-byte aligned", fn,
                    i, k);
      const Range rp = range_of(p, n * pb);
      if (overlap(ro, rp) && !(p == out && pb == ob))
        return fail(TP_ERR_ALIAS, "%s(i=%d): out overlaps peer_partials[%d]", fn, i, k);
      if (overlap(rws, rp))
        return fail(TP_ERR_ALIAS, "%s(i=%d): workspace overlaps peer_partials[%d]", fn, i, k);
      ptrs.p[np++] = p;
    }
    for (int k = np; k < TP_MAX_PARTIALS; ++k) ptrs.p[k] = nullptr;
    if (residual) {
      if (!aligned16(residual))
        return fail(TP_ERR_ALIGNMENT, "%s(i=%d): residual not 16-byte aligned", fn, i);
      const int64_t rb = esize(residual_dtype);
      const Range rr = range_of(residual, n * rb);
      if (overlap(ro, rr) && !(residual == out && rb == ob))
        return fail(TP_ERR_ALIAS, "%s(i=%d): out overlaps the residual", fn, i);
      if (overlap(rws, rr))
        return fail(TP_ERR_ALIAS, "%s(i=%d): workspace overlaps the residual", fn, i);
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const int M = (int)tokens, H = (int)hidden, F = (int)fs;
    const tp::OutType ot = out_dtype == TP_F32 ? tp::OUT_F32 : tp::OUT_BF16;
    auto gemm2_store = [&]() {
      return in_dtype == TP_BF16
                 ? tp::gemm_bf16_store_kb(static_cast<const uint16_t*>(workspace),
                                          tp::gemm_bf16_a_block(M, H, F),
                                          static_cast<const uint16_t*>(W2_i), H, out, H, ot, M,
                                          H, F, split_partials(workspace, M, H, F, in_dtype), s)
                 : tp::gemm_f32(static_cast<const float*>(workspace), F,
                                static_cast<const float*>(W2_i), H, out, H, ot, false, M, H, F,
                                s);
    };
    if (np == 0 && !residual) {  // nothing else to add: the plain shard
      hipError_t e = ffn_gemm1(X, W1_i, ld_w1, workspace, M, H, F, in_dtype, s);
      if (e == hipSuccess) e = gemm2_store();
      return hip_status(e, "tp_ffn_shard_reduce: launch");
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "tp_ffn_shard_reduce: hipGetDevice");
    SideStream* ss = nullptr;
    std::lock_guard<std::mutex> lock(g_side[dev < 0 || dev >= kMaxDevices ? 0 : dev].m);
    e = side_stream(dev, &ss);
    if (e != hipSuccess) return hip_status(e, "tp_ffn_shard_reduce: side stream");
    // S = (other partials, j order) + residual on the side stream, once the
    // caller's stream has reached this call; GEMM1 meanwhile on the caller's.
    e = hipEventRecord(ss->inputs_ready, s);
    if (e == hipSuccess) e = ffn_gemm1(X, W1_i, ld_w1, workspace, M, H, F, in_dtype, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(ss->s, ss->inputs_ready, 0);
    if (e == hipSuccess) {
      if (np > 0)
        e = tp::partial_reduce(ptrs, np, partial_dtype, residual, residual_dtype, S, TP_F32, n,
                               ss->s);
      else {  // only the residual: S = residual in fp32
        ptrs.p[0] = residual;
        e = tp::partial_reduce(ptrs, 1, residual_dtype, nullptr, TP_F32, S, TP_F32, n, ss->s);
      }
    }
    if (e == hipSuccess) e = hipEventRecord(ss->others_summed, ss->s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, ss->others_summed, 0);
    if (e == hipSuccess)
      e = in_dtype == TP_BF16
              ? tp::gemm_bf16_add_kb(static_cast<const uint16_t*>(workspace),
                                     tp::gemm_bf16_a_block(M, H, F),
                                     static_cast<const uint16_t*>(W2_i), H, S, out, H, ot, M, H,
                                     F, split_partials(workspace, M, H, F, in_dtype), s)
              : tp::gemm_f32_add(static_cast<const float*>(workspace), F,
                                 static_cast<const float*>(W2_i), H, S, out, H, ot, M, H, F, s);
    return hip_status(e, "tp_ffn_shard_reduce: launch");
  } catch (...) {
    return fail(TP_ERR_HIP, "tp_ffn_shard_reduce: internal exception");
  }
}

// ---------------------------------------------------------------------------
// Attention shard
// ---------------------------------------------------------------------------
size_t tp_attn_shard_workspace_bytes(int64_t batch, int64_t seq, int32_t n_heads,
                                     int32_t head_dim, int32_t t) {
  if (batch < 0 || seq < 0 || n_heads < 1 || head_dim != kAttnHeadDim || t < 1 || n_heads % t ||
      !attn_shape_ok(batch, seq, n_heads / t))
    return 0;
  return (size_t)attn_layout(batch, seq, n_heads / t, head_dim).total;
}

tp_status_t tp_attn_shard(const void* X, const void* Wqkv_i, const void* Wo_i,
                          void* Y_i, int64_t batch, int64_t seq, int64_t hidden,
                          int32_t n_heads, int32_t head_dim, int32_t i,
                          int32_t t, int32_t causal, int32_t in_dtype,
                          int32_t out_dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  try {
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
      return fail(TP_ERR_DTYPE, "tp_attn_shard: dtype codes in=%d out=%d", in_dtype, out_dtype);
    if (in_dtype != TP_BF16)
      return fail(TP_ERR_UNSUPPORTED, "tp_attn_shard: only bf16 inputs are implemented");
    if (t < 1 || i < 0 || i >= t)
      return fail(TP_ERR_SHARD, "tp_attn_shard: shard i=%d of t=%d", i, t);
    if (batch < 0 || seq < 0 || hidden <= 0 || n_heads < 1 || head_dim < 1 ||
        (causal != 0 && causal != 1))
      return fail(TP_ERR_SHAPE,
                  "tp_attn_shard(i=%d): batch=%lld seq=%lld hidden=%lld n_heads=%d head_dim=%d "
                  "causal=%d",
                  i, (long long)batch, (long long)seq, (long long)hidden, n_heads, head_dim,
                  causal);
    if (n_heads % t != 0)
      return fail(TP_ERR_DIVISIBILITY, "tp_attn_shard(i=%d): n_heads=%d not divisible by t=%d",
                  i, n_heads, t);
    if (head_dim != kAttnHeadDim)
      return fail(TP_ERR_UNSUPPORTED, "tp_attn_shard(i=%d): head_dim=%d (only 128)", i, head_dim);
    if (hidden % 8 != 0)
      return fail(TP_ERR_SHAPE, "tp_attn_shard(i=%d): hidden=%lld must be a multiple of 8", i,
                  (long long)hidden);
    const int64_t nl = n_heads / t;
    if (hidden >= kMaxLdA || !attn_shape_ok(batch, seq, nl))
      return fail(TP_ERR_SHAPE,
                  "tp_attn_shard(i=%d): needs batch*seq and batch*(n_heads/t)*ceil(seq/64) "
                  "within 2^31-1, hidden and 2*(n_heads/t)*head_dim below 2^22 and seq below "
                  "2^23 (batch=%lld seq=%lld hidden=%lld n_heads/t=%lld)",
                  i, (long long)batch, (long long)seq, (long long)hidden, (long long)nl);
    const int64_t tokens = batch * seq;
    if (tokens == 0) return ok();
    if (!X || !Wqkv_i || !Wo_i || !Y_i)
      return fail(TP_ERR_NULL, "tp_attn_shard(i=%d): NULL tensor pointer", i);
    if (!workspace) return fail(TP_ERR_WORKSPACE, "tp_attn_shard(i=%d): NULL workspace", i);
    if (!aligned16(X) || !aligned16(Wqkv_i) || !aligned16(Wo_i) || !aligned16(Y_i) ||
        !aligned16(workspace))
      return fail(TP_ERR_ALIGNMENT, "tp_attn_shard(i=%d): pointers must be 16-byte aligned", i);
    const AttnLayout L = attn_layout(batch, seq, nl, head_dim);
    if (workspace_bytes < (size_t)L.total)
      return fail(TP_ERR_WORKSPACE, "tp_attn_shard(i=%d): workspace %zu bytes < %lld needed", i,
                  workspace_bytes, (long long)L.total);
    const int64_t nqkv = 3 * nl * head_dim;
    const Range rx = range_of(X, tokens * hidden * 2);
    const Range rq = range_of(Wqkv_i, hidden * nqkv * 2);
    const Range ro = range_of(Wo_i, nl * head_dim * hidden * 2);
    const Range ry = range_of(Y_i, tokens * hidden * esize(out_dtype));
    const Range rws = range_of(workspace, L.total);
    if (overlap(ry, rx) || overlap(ry, rq) || overlap(ry, ro) || overlap(ry, rws))
      return fail(TP_ERR_ALIAS, "tp_attn_shard(i=%d): Y_i overlaps an input or the workspace", i);
    if (overlap(rws, rx) || overlap(rws, rq) || overlap(rws, ro))
      return fail(TP_ERR_ALIAS, "tp_attn_shard(i=%d): workspace overlaps an input", i);

    uint8_t* ws = static_cast<uint8_t*>(workspace);
    tp::QkvOut q;
    q.q = reinterpret_cast<uint16_t*>(ws + 0 * L.part_bytes);
    q.k = reinterpret_cast<uint16_t*>(ws + 1 * L.part_bytes);
    q.vt_hi = reinterpret_cast<uint16_t*>(ws + 2 * L.part_bytes);
    q.vt_lo = reinterpret_cast<uint16_t*>(ws + 3 * L.part_bytes);
    q.seq = (int32_t)seq;
    q.seq_pad = (int32_t)L.seq_pad;
    q.nl = (int32_t)nl;
    q.d = head_dim;
    uint16_t* O = reinterpret_cast<uint16_t*>(ws + kAttnParts * L.part_bytes);

    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    hipError_t e = tp::gemm_bf16_qkv(static_cast<const uint16_t*>(X), hidden,
                                     static_cast<const uint16_t*>(Wqkv_i), nqkv, q,
                                     (int)tokens, (int)nqkv, (int)hidden, s);
    if (e != hipSuccess) return hip_status(e, "tp_attn_shard: QKV launch");
    float* part = reinterpret_cast<float*>(ws + kAttnParts * L.part_bytes + L.o_bytes);
    // O is written in the layout the output projection reads (fp16 O_hi
    // K-blocked by its stage depth, then the bf8 residual O_lo K-blocked by
    // the lo product's 64), so each of its A stages is one contiguous run.
    e = tp::attention_fwd(q, (int)batch, causal != 0, O, part, s);
    if (e != hipSuccess) return hip_status(e, "tp_attn_shard: attention launch");
    e = tp::gemm_f16_bf8_store_kb(reinterpret_cast<const uint8_t*>(O),
                                  static_cast<const uint16_t*>(Wo_i), hidden, Y_i, hidden,
                                  out_dtype == TP_F32 ? tp::OUT_F32 : tp::OUT_BF16, (int)tokens,
                                  (int)hidden, (int)(nl * head_dim), s);
    if (e != hipSuccess) return hip_status(e, "tp_attn_shard: output projection launch");
    return ok();
  } catch (...) {
    return fail(TP_ERR_HIP, "tp_attn_shard: internal exception");
  }
}

// ---------------------------------------------------------------------------
// Partial reduce
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

tp_status_t reduce_checked(const char* fn, const void* const* partials, int32_t t,
                          const void* residual, void* out, int64_t rows, int64_t cols,
                          int32_t partial_dtype, int32_t residual_dtype, int32_t out_dtype,
                          void* stream) {
  try {
    if (!valid_dtype(partial_dtype) || !valid_dtype(out_dtype) ||
        (residual && !valid_dtype(residual_dtype)))
      return fail(TP_ERR_DTYPE, "%s: dtype codes p=%d r=%d o=%d", fn, partial_dtype,
                  residual_dtype, out_dtype);
    if (t < 1 || t > TP_MAX_PARTIALS)
      return fail(TP_ERR_SHARD, "%s: t=%d outside [1, %d]", fn, t, TP_MAX_PARTIALS);
    if (rows < 0 || cols < 0 || cols % 8 != 0 ||
        (rows > 0 && cols > (int64_t(1) << 60) / rows))
      return fail(TP_ERR_SHAPE,
                  "%s: rows=%lld cols=%lld (cols a multiple of 8, rows*cols at most 2^60)",
                  fn, (long long)rows, (long long)cols);
    const int64_t n = rows * cols;
    if (n == 0) return ok();
    if (!partials || !out) return fail(TP_ERR_NULL, "%s: NULL pointer", fn);
    tp::ReducePtrs ptrs;
    for (int k = 0; k < t; ++k) {
      if (!partials[k]) return fail(TP_ERR_NULL, "%s: partials[%d] is NULL", fn, k);
      if (!aligned16(partials[k]))
        return fail(TP_ERR_ALIGNMENT, "%s: partials[%d] not 16-byte aligned", fn, k);
      ptrs.p[k] = partials[k];
    }
    for (int k = t; k < TP_MAX_PARTIALS; ++k) ptrs.p[k] = nullptr;
    if (!aligned16(out) || (residual && !aligned16(residual)))
      return fail(TP_ERR_ALIGNMENT, "%s: pointers must be 16-byte aligned", fn);
    // out may be exactly one of the inputs (same address, same element size):
    // every element group is read in full by the thread that writes it.
    const int64_t ob = esize(out_dtype);
    const Range ro = range_of(out, n * ob);
    for (int k = 0; k < t; ++k) {
      const int64_t pb = esize(partial_dtype);
      if (overlap(ro, range_of(partials[k], n * pb)) && !(partials[k] == out && pb == ob))
        return fail(TP_ERR_ALIAS, "%s: out overlaps partials[%d]", fn, k);
    }
    if (residual) {
      const int64_t rb = esize(residual_dtype);
      if (overlap(ro, range_of(residual, n * rb)) && !(residual == out && rb == ob))
        return fail(TP_ERR_ALIAS, "%s: out overlaps the residual", fn);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const hipError_t e = tp::partial_reduce(ptrs, t, partial_dtype, residual, residual_dtype,
                                            out, out_dtype, n, s);
    return hip_status(e, fn);
  } catch (...) {
    return fail(TP_ERR_HIP, "%s: internal exception", fn);
  }
}

}  // namespace

extern "C" {

tp_status_t tp_partial_reduce(const void* const* partials, int32_t t,
                              const void* residual, void* out, int64_t rows,
                              int64_t cols, int32_t partial_dtype,
                              int32_t residual_dtype, int32_t out_dtype,
                              void* stream) {
  return reduce_checked("tp_partial_reduce", partials, t, residual, out, rows, cols,
                        partial_dtype, residual_dtype, out_dtype, stream);
}

tp_status_t tp_partial_reduce_slice(const void* const* partials, int32_t t,
                                    const void* residual, void* out, int64_t rows,
                                    int64_t cols, int32_t slice, int32_t nslices,
                                    int32_t partial_dtype, int32_t residual_dtype,
                                    int32_t out_dtype, void* stream) {
  const char* fn = "tp_partial_reduce_slice";
  try {
    if (!valid_dtype(partial_dtype) || !valid_dtype(out_dtype) ||
        (residual && !valid_dtype(residual_dtype)))
      return fail(TP_ERR_DTYPE, "%s: dtype codes p=%d r=%d o=%d", fn, partial_dtype,
                  residual_dtype, out_dtype);
    if (t < 1 || t > TP_MAX_PARTIALS)
      return fail(TP_ERR_SHARD, "%s: t=%d outside [1, %d]", fn, t, TP_MAX_PARTIALS);
    if (nslices < 1 || slice < 0 || slice >= nslices)
      return fail(TP_ERR_SHARD, "%s: slice %d of %d", fn, slice, nslices);
    if (rows < 0 || cols < 0 || (rows > 0 && cols > (int64_t(1) << 60) / rows))
      return fail(TP_ERR_SHAPE, "%s: rows=%lld cols=%lld (rows*cols at most 2^60)", fn,
                  (long long)rows, (long long)cols);
    // balanced row blocks: the first rows % nslices slices hold one more row
    const int64_t base = rows / nslices, extra = rows % nslices;
    const int64_t r0 = slice * base + (slice < extra ? slice : extra);
    const int64_t r1 = r0 + base + (slice < extra ? 1 : 0);
    if (r1 == r0 || cols == 0) return reduce_checked(fn, partials, t, residual, out, 0, cols,
                                                     partial_dtype, residual_dtype, out_dtype,
                                                     stream);
    if (!partials || !out) return fail(TP_ERR_NULL, "%s: NULL pointer", fn);
    const int64_t off = r0 * cols;
    const void* p[TP_MAX_PARTIALS];
    for (int k = 0; k < t; ++k) {
      if (!partials[k]) return fail(TP_ERR_NULL, "%s: partials[%d] is NULL", fn, k);
      p[k] = static_cast<const char*>(partials[k]) + off * esize(partial_dtype);
    }
    const void* r =
        residual ? static_cast<const char*>(residual) + off * esize(residual_dtype) : nullptr;
    void* o = static_cast<char*>(out) + off * esize(out_dtype);
    return reduce_checked(fn, p, t, r, o, r1 - r0, cols, partial_dtype, residual_dtype,
                          out_dtype, stream);
  } catch (...) {
    return fail(TP_ERR_HIP, "%s: internal exception", fn);
  }
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Sequence-parallel sum + LayerNorm
// ---------------------------------------------------------------------------
extern "C" {

tp_status_t tp_sp_reduce_layernorm(const void* const* partials, int32_t t, const void* residual,
                                   void* x_out, void* ln_out, const float* gamma,
                                   const float* beta, float eps, int64_t rows, int64_t cols,
                                   int32_t slice, int32_t nslices, int32_t partial_dtype,
                                   int32_t residual_dtype, int32_t x_dtype, int32_t ln_dtype,
                                   void* stream) {
  const char* fn = "tp_sp_reduce_layernorm";
  try {
    if (!valid_dtype(partial_dtype) || !valid_dtype(ln_dtype) ||
        (residual && !valid_dtype(residual_dtype)) || (x_out && !valid_dtype(x_dtype)))
      return fail(TP_ERR_DTYPE, "%s: dtype codes p=%d r=%d x=%d y=%d", fn, partial_dtype,
                  residual_dtype, x_dtype, ln_dtype);
    if (t < 1 || t > TP_MAX_PARTIALS)
      return fail(TP_ERR_SHARD, "%s: t=%d outside [1, %d]", fn, t, TP_MAX_PARTIALS);
    if (nslices < 1 || slice < 0 || slice >= nslices)
      return fail(TP_ERR_SHARD, "%s: slice %d of %d", fn, slice, nslices);
    if (rows < 0 || cols < 0 || cols % 8 != 0 || cols > tp::kLnMaxCols ||
        (rows > 0 && cols > (int64_t(1) << 60) / rows))
      return fail(TP_ERR_SHAPE,
                  "%s: rows=%lld cols=%lld (cols a multiple of 8, at most %d)", fn,
                  (long long)rows, (long long)cols, tp::kLnMaxCols);
    if (!(eps >= 0.0f) || eps > 3.0e38f)
      return fail(TP_ERR_SHAPE, "%s: eps=%g must be finite and >= 0", fn, (double)eps);
    const int64_t base = rows / nslices, extra = rows % nslices;
    const int64_t r0 = slice * base + (slice < extra ? slice : extra);
    const int64_t nr = base + (slice < extra ? 1 : 0);
    if (nr == 0 || cols == 0) return ok();
    if (!partials || !ln_out) return fail(TP_ERR_NULL, "%s: NULL pointer", fn);
    const int64_t pb = esize(partial_dtype), yb = esize(ln_dtype);
    const int64_t n = rows * cols;
    tp::ReducePtrs ptrs;
    for (int k = 0; k < t; ++k) {
      if (!partials[k]) return fail(TP_ERR_NULL, "%s: partials[%d] is NULL", fn, k);
      if (!aligned16(partials[k]))
        return fail(TP_ERR_ALIGNMENT, "%s: partials[%d] not 16-byte aligned", fn, k);
      ptrs.p[k] = static_cast<const char*>(partials[k]) + r0 * cols * pb;
    }
    for (int k = t; k < TP_MAX_PARTIALS; ++k) ptrs.p[k] = nullptr;
    if (!aligned16(ln_out) || (residual && !aligned16(residual)) ||
        (x_out && !aligned16(x_out)) || (gamma && !aligned16(gamma)) ||
        (beta && !aligned16(beta)))
      return fail(TP_ERR_ALIGNMENT, "%s: pointers must be 16-byte aligned", fn);
    // ln_out overlaps nothing; x_out may be exactly one of the inputs of the
    // same element size (each row is read in full before it is written)
    const Range ry = range_of(ln_out, n * yb);
    const int64_t rb = esize(residual_dtype), xb = esize(x_dtype);
    for (int k = 0; k < t; ++k) {
      const Range rp = range_of(partials[k], n * pb);
      if (overlap(ry, rp)) return fail(TP_ERR_ALIAS, "%s: ln_out overlaps partials[%d]", fn, k);
      if (x_out && overlap(range_of(x_out, n * xb), rp) && !(partials[k] == x_out && pb == xb))
        return fail(TP_ERR_ALIAS, "%s: x_out overlaps partials[%d]", fn, k);
    }
    if (residual) {
      const Range rr = range_of(residual, n * rb);
      if (overlap(ry, rr)) return fail(TP_ERR_ALIAS, "%s: ln_out overlaps the residual", fn);
      if (x_out && overlap(range_of(x_out, n * xb), rr) && !(residual == x_out && rb == xb))
        return fail(TP_ERR_ALIAS, "%s: x_out overlaps the residual", fn);
    }
    if (x_out && overlap(ry, range_of(x_out, n * xb)))
      return fail(TP_ERR_ALIAS, "%s: ln_out overlaps x_out", fn);
    if ((gamma && overlap(ry, range_of(gamma, cols * 4))) ||
        (beta && overlap(ry, range_of(beta, cols * 4))) ||
        (x_out && gamma && overlap(range_of(x_out, n * xb), range_of(gamma, cols * 4))) ||
        (x_out && beta && overlap(range_of(x_out, n * xb), range_of(beta, cols * 4))))
      return fail(TP_ERR_ALIAS, "%s: an output overlaps gamma or beta", fn);
    const void* R = residual ? static_cast<const char*>(residual) + r0 * cols * rb : nullptr;
    void* X = x_out ? static_cast<char*>(x_out) + r0 * cols * xb : nullptr;
    void* Y = static_cast<char*>(ln_out) + r0 * cols * yb;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const hipError_t e = tp::reduce_layernorm(ptrs, t, partial_dtype, R, residual_dtype, X,
                                              x_dtype, Y, ln_dtype, gamma, beta, eps, nr,
                                              (int)cols, s);
    return hip_status(e, fn);
  } catch (...) {
    return fail(TP_ERR_HIP, "%s: internal exception", fn);
  }
}

}  // extern "C"
