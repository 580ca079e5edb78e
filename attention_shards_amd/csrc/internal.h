// Internal declarations shared by the host dispatch (tp_shard.cpp) and the
// HIP kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

// Output element type of a GEMM epilogue.
enum OutType { OUT_F32 = 0, OUT_BF16 = 1 };

// Where the QKV projection's epilogue scatters its columns.  All buffers are
// 16-bit words.  Q and K are [batch][nl][seq_pad][d] (d contiguous), each a
// bf16 hi/lo pair: hi = bf16(v), lo = bf16(v - hi).  V is stored transposed,
// [batch][nl][d][seq_pad] (sequence contiguous), because it is the row
// operand of the probability-times-value product, as an fp16 hi/lo pair
// (the probabilities are fp16).
struct QkvOut {
  uint16_t* q_hi;
  uint16_t* q_lo;
  uint16_t* k_hi;
  uint16_t* k_lo;
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
// K block the kernel chosen for an [M, N] output reads a K-blocked A in.
int gemm_bf16_a_block(int M, int N);
// C = acc stored as `out` (row stride ldc), A K-blocked, [ceil(K/kb)][M][kb];
// kb must be gemm_bf16_a_block(M, N) (else hipErrorInvalidValue).
hipError_t gemm_bf16_store_kb(const uint16_t* A, int kb, const uint16_t* B, int64_t ldb,
                              void* C, int64_t ldc, OutType out, int M, int N, int K,
                              hipStream_t s);
// C = [A_hi | A_lo] * B: A2 is [M, 2K], the same B[K,N] multiplies both
// halves (two MFMA passes over K); K a multiple of 64; A2 K-blocked,
// [2K/kb][M][kb], kb = gemm_bf16_a_block(M, N).
hipError_t gemm_bf16_store_split_a_kb(const uint16_t* A2, int kb, const uint16_t* B,
                                      int64_t ldb, void* C, int64_t ldc, OutType out, int M,
                                      int N, int K, hipStream_t s);
// Same product scattered into the attention workspace (N == 3*nl*d).
hipError_t gemm_bf16_qkv(const uint16_t* A, int64_t lda, const uint16_t* B,
                         int64_t ldb, const QkvOut& q, int M, int N, int K,
                         hipStream_t s);

// fp32 inputs, fp32 MFMA.  Requirements: K % 4 == 0, N % 4 == 0.
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

// Causal / full attention over the QKV workspace; writes O as a bf16 hi/lo
// pair [batch*seq, 2*nl*d]: O_hi in columns [0, nl*d), O_lo in
// [nl*d, 2*nl*d), row-major for o_kb == 0 or K-blocked for the output
// projection, [2*nl*d/o_kb][batch*seq][o_kb] (o_kb = 32 or 64).  d must be
// 128.  `part` (attn_partial_bytes, 16-byte aligned) holds the partial
// results of split query blocks.
hipError_t attention_fwd(const QkvOut& q, int batch, bool causal, uint16_t* O, int o_kb,
                         float* part, hipStream_t s);

// out = sum_i P_i + R, fp32 accumulate, any n (the last n % 8 elements take
// a scalar path).
struct ReducePtrs {
  const void* p[64];
};
hipError_t partial_reduce(const ReducePtrs& ptrs, int t, int pdt,
                          const void* R, int rdt, void* out, int odt,
                          int64_t n, hipStream_t s);

// C = S + A*B: the product added to an fp32 [M, N] matrix S (row stride
// ldc, like C) and rounded once to the output type.  bf16 (A K-blocked as
// for gemm_bf16_store_kb) and fp32 inputs (requirements of gemm_f32).
hipError_t gemm_bf16_add_kb(const uint16_t* A, int kb, const uint16_t* B, int64_t ldb,
                            const float* S, void* C, int64_t ldc, OutType out, int M, int N,
                            int K, hipStream_t s);
hipError_t gemm_f32_add(const float* A, int64_t lda, const float* B, int64_t ldb,
                        const float* S, void* C, int64_t ldc, OutType out, int M, int N,
                        int K, hipStream_t s);

}  // namespace tp
