// Internal declarations shared by the host dispatch (tp_shard.cpp) and the
// HIP kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tp_shard.h"

namespace tp {

// Compute units of the current device (hipDeviceAttributeMultiprocessorCount,
// cached per device); 256 (a full MI355X) when no device can be queried.
// The tile and work-split choices size their waves of workgroups by it.
int device_cu_count();

// Output element type of a GEMM epilogue.
enum OutType { OUT_F32 = 0, OUT_BF16 = 1 };

// Where the QKV projection's epilogue scatters its columns.  All buffers are
// 16-bit words.  Q and K are fp16, [batch][nl][seq_pad][d] (d contiguous).
// V is stored transposed, [batch][nl][d][seq_pad] (sequence contiguous),
// because it is the row operand of the probability-times-value product, as
// an fp16 hi/lo pair (the probabilities are fp16): hi = fp16(v),
// lo = fp16(v - hi).
struct QkvOut {
  uint16_t* q;
  uint16_t* k;
  uint16_t* vt_hi;
  uint16_t* vt_lo;
  int32_t seq;      // tokens per sequence
  int32_t seq_pad;  // seq rounded up to the attention key tile (64)
  int32_t nl;       // local heads
  int32_t d;        // head dim
};

// bf16 products C[M,N] = A[M,K] * B[K,N] with fp32 accumulation.  A is
// K-contiguous (row stride lda, or K-blocked where stated), B is
// N-contiguous (row stride ldb).  Requirements checked by the caller:
// K % 8 == 0, N % 8 == 0, lda/ldb % 8 == 0, 16-byte aligned A and B.
//
// C = bf16(GeLU_erf(acc)): row-major (row stride ldc) for
// kb == 0, else K-blocked for a following product, [ceil(N/kb)][M][kb]
// (kb = 32 or 64; columns past N in the last block are not written).
hipError_t gemm_bf16_gelu(const uint16_t* A, int64_t lda, const uint16_t* B,
                          int64_t ldb, uint16_t* C, int64_t ldc, int M, int N,
                          int K, int kb, hipStream_t s);
// The same with A already K-blocked, [ceil(K/kb)][M][kb], kb =
// gemm_bf16_a_block(M, N, 0) (else hipErrorInvalidValue); C K-blocked by
// kb_out (32 or 64).
hipError_t gemm_bf16_gelu_akb(const uint16_t* Akb, int kb, const uint16_t* B, int64_t ldb,
                              uint16_t* C, int M, int N, int K, int kb_out, hipStream_t s);
// A [M, K] row-major (row stride lda) copied K-blocked into out,
// [ceil(K/kb)][M][kb] (kb = 32 or 64), zeros past K.  K, lda multiples of 8.
hipError_t kblock_bf16(const uint16_t* A, int64_t lda, uint16_t* out, int M, int K, int kb,
                       hipStream_t s);
// K block the kernel chosen for an [M, N] output reads a K-blocked A in;
// k_split: K when the product is given fp32 partials for a split K (the
// plan may then differ), else 0.
int gemm_bf16_a_block(int M, int N, int64_t k_split);
// Bytes of fp32 partials an [M, N] product over K may split K into (0: the
// plan does not split it).
int64_t gemm_bf16_split_bytes(int M, int N, int64_t K);
// C = acc stored as `out` (row stride ldc), A K-blocked, [ceil(K/kb)][M][kb];
// kb must be gemm_bf16_a_block(M, N, partials ? K : 0) (else
// hipErrorInvalidValue).  partials: nullptr, or gemm_bf16_split_bytes(M, N,
// K) bytes (256-byte aligned) the call may use to split K.
hipError_t gemm_bf16_store_kb(const uint16_t* A, int kb, const uint16_t* B, int64_t ldb,
                              void* C, int64_t ldc, OutType out, int M, int N, int K,
                              float* partials, hipStream_t s);
// C = A_hi * fp16(B) + A_lo * bf8(B) in one pass over K, B bf16 (converted
// in registers), A as attention_fwd writes O: A_hi fp16 K-blocked by 32,
// then A_lo bf8 K-blocked by 64 with permuted row pieces (3*K*M bytes); K a
// multiple of 64.  Every stage brings A_hi's and B's tiles, every second
// stage also A_lo's tile for two stages; the lo product runs 32x32x64 bf8
// MFMAs (twice the fp16 rate).
hipError_t gemm_f16_bf8_store_kb(const uint8_t* A, const uint16_t* B, int64_t ldb, void* C,
                                 int64_t ldc, OutType out, int M, int N, int K, hipStream_t s);
// Same product scattered into the attention workspace (N == 3*nl*d).
hipError_t gemm_bf16_qkv(const uint16_t* A, int64_t lda, const uint16_t* B,
                         int64_t ldb, const QkvOut& q, int M, int N, int K,
                         hipStream_t s);

// fp32 inputs, fp32 MFMA.  Requirements: K % 4 == 0, N % 4 == 0; with gelu the
// output is fp32 (GeLU(Z) is kept in fp32 between the fp32 products).
hipError_t gemm_f32(const float* A, int64_t lda, const float* B, int64_t ldb,
                    void* C, int64_t ldc, OutType out, bool gelu, int M, int N,
                    int K, hipStream_t s);

// How the attention kernel splits its work: query blocks of 128, key ranges
// cut into chunks of `ch` tiles of 64 keys, one workgroup per (query block,
// chunk, sequence*head).  The same function sizes the workspace and
// launches the kernel.
struct AttnSplit {
  int32_t qb;       // queries per block (128 or 256)
  int32_t nqb;      // query blocks per sequence
  int32_t ch;       // key tiles per chunk
  int32_t n_items;  // workgroups of the attention kernel
  int32_t nbh;      // batch * local heads
};
AttnSplit attn_split(int batch, int seq, int nl, bool causal);
// Bytes for the chunks' partial results (the larger of causal and full).
int64_t attn_partial_bytes(int batch, int seq, int nl);

// Causal / full attention over the QKV workspace; writes O [batch*seq,
// nl*d] for the output projection (gemm_f16_bf8_store_kb) as O_hi = fp16(O),
// K-blocked by 32, [nl*d/32][batch*seq][32], followed by O_lo = bf8(O -
// O_hi), K-blocked by 64, [nl*d/64][batch*seq][64 bytes], each 64-byte row
// piece permuted (byte 32h + 8s + j holds column 16s + 8h + j): 3 bytes per
// element in all.  d must be 128.  `part` (attn_partial_bytes, 16-byte
// aligned) holds the partial results of split query blocks.
hipError_t attention_fwd(const QkvOut& q, int batch, bool causal, uint16_t* O, float* part,
                         hipStream_t s);

// out = sum_i P_i + R, fp32 accumulate, any n (the last n % 8 elements take
// a scalar path).
struct ReducePtrs {
  const void* p[64];
};
hipError_t partial_reduce(const ReducePtrs& ptrs, int t, int pdt,
                          const void* R, int rdt, void* out, int odt,
                          int64_t n, hipStream_t s);

// Rows [0, rows) of x = sum_i P_i + R (fp32, fixed order; R nullable) and
// y = LayerNorm(x) per row: (x - mean) / sqrt(var + eps) * gamma + beta,
// biased variance, gamma/beta fp32 [cols] (nullable: 1 and 0).  xout is
// nullable (x not stored).  cols a multiple of 8, at most kLnMaxCols.
constexpr int kLnMaxCols = 512 * 8 * 8;  // 512 threads x 8 groups x 8 columns
hipError_t reduce_layernorm(const ReducePtrs& ptrs, int t, int pdt, const void* R, int rdt,
                            void* xout, int xdt, void* yout, int ydt, const float* gamma,
                            const float* beta, float eps, int64_t rows, int cols,
                            hipStream_t s);

// C = S + A*B: the product added to an fp32 [M, N] matrix S (row stride
// ldc, like C) and rounded once to the output type.  bf16 (A K-blocked and
// partials as for gemm_bf16_store_kb) and fp32 inputs (requirements of
// gemm_f32).
hipError_t gemm_bf16_add_kb(const uint16_t* A, int kb, const uint16_t* B, int64_t ldb,
                            const float* S, void* C, int64_t ldc, OutType out, int M, int N,
                            int K, float* partials, hipStream_t s);
hipError_t gemm_f32_add(const float* A, int64_t lda, const float* B, int64_t ldb,
                        const float* S, void* C, int64_t ldc, OutType out, int M, int N,
                        int K, hipStream_t s);

// The argument checks of tp_ffn_shard without the workspace ones (for an
// entry point that supplies its own memory); sets the error message.
tp_status_t ffn_check_args(const char* fn, const void* X, const void* W1_i, const void* W2_i,
                           const void* Y_i, int64_t tokens, int64_t hidden, int64_t ffn,
                           int32_t i, int32_t t, int64_t ld_w1, int32_t in_dtype,
                           int32_t out_dtype);
// Records `msg` as the thread's last error and returns st.
tp_status_t set_error(tp_status_t st, const char* msg);

}  // namespace tp
