// Dense GEMMs of the shard path on gfx950 matrix cores.
//
//   bf16:  C[M,N] = A[M,K] * B[K,N], v_mfma_f32_32x32x16_bf16, fp32 accumulators.
//   fp32:  the same product with v_mfma_f32_16x16x4_f32.
//
// They serve the column-parallel W1 product with its element-wise GeLU
// epilogue, the row-parallel W2 product, the head-sharded QKV projection and
// the row-parallel output projection (page "Tensor Parallelism > Combining
// Column and Row Parallelism", FFN steps 1-2 and the attention paragraphs).
//
// bf16 kernels
//   * Both operands go from memory straight into an LDS ring with buffer
//     loads that write LDS (1 KiB per instruction), tracked with explicit
//     vmcnt waits.  A (activations, K-contiguous) is stored as K-rows with a
//     16-byte-chunk XOR swizzle and read with ds_read_b128; B (weights,
//     N-contiguous) keeps its [k][n] layout with a 64-byte-block swizzle and
//     is read with ds_read_b64_tr_b16, which transposes it into the MFMA
//     operand.
//   * gemm_bf16_kernel: 4 waves (one per SIMD), DMAs and fragment reads
//     interleaved between the MFMAs of each wave.  256x256 tiles: each wave
//     owns a 128x128 block (256 accumulator registers), K = 32 per stage
//     through a 5-slot ring (160 KB) over a K-blocked A; the wide wave block
//     halves the LDS fragment reads per MFMA of a 128x64 block.  256x192
//     tiles: 128x96 per wave, K = 32 per stage, five 28 KB slots.  256x128,
//     128x192 and 128x128 tiles: K = 64 per stage through a 3-slot ring.
//     (128x192 fills all 256 CUs where 256x128 would leave a quarter idle,
//     e.g. 2048 x 3072 outputs.)  The K = 32 kinds over a row-major A keep A
//     in two slots of 128-byte rows, each the K columns of two stages,
//     beside a 4-slot B ring, so that A's DMAs read whole lines of its rows.
//   * A tile plan covers the output with whole waves of one kind and, where
//     that leaves a wave partly idle, the remaining columns in a second kind
//     (two launches).
//   * Epilogues run on the fp32 accumulators staged through LDS: GeLU to
//     bf16 (a fit accurate to well below bf16's rounding) or, for the fp32
//     products, to fp32; plain stores; the Q/K/V^T scatter of the attention
//     workspace; the add of a pre-summed fp32 matrix.
//   * Workgroup ids are remapped so each XCD (dispatch is round-robin over
//     the 8 XCDs) receives a contiguous run of tiles, ordered in groups of 8
//     tile-rows so neighbouring tiles share A and B panels in that XCD's L2.
#include <algorithm>
#include <atomic>
#include <numeric>
#include <type_traits>

#include "internal.h"

namespace tp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Two fp32 values rounded to bf16 (nearest even) and packed, low half
// first: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// GeLU(z) = z * Phi(z), Phi the standard normal CDF, with Phi from erfc
// through the Chebyshev fit of Press, Teukolsky, Vetterling and Flannery,
// Numerical Recipes (2nd ed.), section 6.2, function erfcc:
//     erfc(x) = t exp(-x^2 + P(t)),  t = 1/(1 + x/2),  P of degree 9,
// with a fractional error below 1.2e-7 for every x >= 0, so the value stays
// relatively accurate deep in the negative tail (z = -12: Phi ~ 2e-33).
// Taken at x = |z|/sqrt(2) and written in base 2 (the coefficients are
// P's times log2(e)).  With E = z erfc(x)/2 (the sign of z), GeLU = z - E
// for z >= 0 and E for z < 0, i.e. max(z, 0) - |E|.  Branch-free: one
// reciprocal, one exponential, fifteen multiply(-add)s, a max and a
// subtract.  Evaluated in fp32 (hardware rcp/exp2): |error| <= 2.5e-7 |z|,
// relative error <= 1e-5.
__device__ __forceinline__ float gelu_erf(float z) {
  constexpr double L2E = 1.4426950408889634;
  constexpr float C0 = (float)(-1.26551223 * L2E), C1 = (float)(1.00002368 * L2E),
                  C2 = (float)(0.37409196 * L2E), C3 = (float)(0.09678418 * L2E),
                  C4 = (float)(-0.18628806 * L2E), C5 = (float)(0.27886807 * L2E),
                  C6 = (float)(-1.13520398 * L2E), C7 = (float)(1.48851587 * L2E),
                  C8 = (float)(-0.82215223 * L2E), C9 = (float)(0.17087277 * L2E);
  // t = 1 / (1 + x/2) with x = |z| / sqrt(2)
  const float t = __builtin_amdgcn_rcpf(fmaf(fabsf(z), 0.35355339059327376f, 1.0f));
  float p = fmaf(C9, t, C8);
  p = fmaf(p, t, C7);
  p = fmaf(p, t, C6);
  p = fmaf(p, t, C5);
  p = fmaf(p, t, C4);
  p = fmaf(p, t, C3);
  p = fmaf(p, t, C2);
  p = fmaf(p, t, C1);
  p = fmaf(p, t, C0);
  // exp(-x^2 + P) = exp2(log2(e) (-z^2/2) + log2(e) P)
  const float e = __builtin_amdgcn_exp2f(fmaf(z, z * (float)(-0.5 * L2E), p));
  const float E = (0.5f * z) * t * e;
  return fmaxf(z, 0.0f) - fabsf(E);
}

// GeLU(z) for a result rounded to bf16 (8-bit significand: an error well
// below half a unit in the last place, 2^-9 relative, leaves at most one
// unit after rounding).  Same form as gelu_erf with P replaced by Q of
// degree 5, the minimax (Remez) fit of log2(erfc(x) exp(x^2) / t) - 1 over
// t in [0.17, 1], i.e. |z| <= 13.8: erfc(x)/2 = t exp2(-x^2 log2(e) + Q(t)).
// Q's maximum error is 1.1e-5 in base-2 units (7.6e-6 relative); with the
// fp32 rounding of the exponent's argument (up to 104 in size at z = -12)
// the GeLU's relative error stays below 1.2e-5 for |z| <= 12 and 1.4e-5
// down to z = -13 (below about -13.06 the exponential leaves the normal fp32
// range; the exact GeLU is 3.6e-38 there).  GeLU = max(z, 0) - (|z| t)
// exp2(...) as one fused multiply-add: one reciprocal, one exponential and
// eleven other vector operations (gelu_erf: seventeen).
__device__ __forceinline__ float gelu_erf_bf16(float z) {
  constexpr double L2E = 1.4426950408889634;
  constexpr float Q0 = -2.827233510302323f, Q1 = 1.468683049078055f,
                  Q2 = 0.3670840868812766f, Q3 = 0.6845487657077611f,
                  Q4 = -1.0231460297394164f, Q5 = 0.33007462354023553f;
  const float t = __builtin_amdgcn_rcpf(fmaf(fabsf(z), 0.35355339059327376f, 1.0f));
  float q = fmaf(Q5, t, Q4);
  q = fmaf(q, t, Q3);
  q = fmaf(q, t, Q2);
  q = fmaf(q, t, Q1);
  q = fmaf(q, t, Q0);
  const float e = __builtin_amdgcn_exp2f(fmaf(z, z * (float)(-0.5 * L2E), q));
  // max(z, 0) as an integer max of the bits (a set sign bit is a negative
  // integer): one instruction, where fmaxf first canonicalizes z
  const int zb = __builtin_bit_cast(int, z);
  const float zpos = __builtin_bit_cast(float, zb > 0 ? zb : 0);
  return fmaf(-(fabsf(z) * t), e, zpos);
}

// ---------------------------------------------------------------------------
// Epilogues: store4 receives four accumulators of columns col0..col0+3 of one
// row (col0 % 4 == 0; the caller has checked row < M and col0 < N, and N % 4
// == 0 so the run is entirely inside the matrix).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_run4(void* C, int64_t ldc, int out, int row,
                                           int col0, const float* v) {
  if (out == OUT_F32) {
    float* c = static_cast<float*>(C) + (int64_t)row * ldc + col0;
    *reinterpret_cast<f32x4*>(c) = f32x4{v[0], v[1], v[2], v[3]};
  } else {
    uint16_t* c = static_cast<uint16_t*>(C) + (int64_t)row * ldc + col0;
    *reinterpret_cast<uint2*>(c) = uint2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
  }
}

// 8 consecutive columns (col0 % 8 == 0, the run inside the matrix).
__device__ __forceinline__ void store_run8(void* C, int64_t ldc, int out, int row,
                                           int col0, const float* v) {
  if (out == OUT_F32) {
    f32x4* c = reinterpret_cast<f32x4*>(static_cast<float*>(C) + (int64_t)row * ldc + col0);
    c[0] = f32x4{v[0], v[1], v[2], v[3]};
    c[1] = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    uint16_t* c = static_cast<uint16_t*>(C) + (int64_t)row * ldc + col0;
    *reinterpret_cast<u32x4*>(c) = u32x4{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]),
                                         pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
  }
}

struct EpiStore {
  void* C;
  int64_t ldc;
  int out;  // OutType
  __device__ void store4(int row, int col0, const float* v) const {
    store_run4(C, ldc, out, row, col0, v);
  }
  __device__ void store8(int row, int col0, const float* v) const {
    store_run8(C, ldc, out, row, col0, v);
  }
};

// GeLU(acc) rounded to bf16, row-major (row stride ldc) or, with
// kb_shift > 0, K-blocked for the next product: column c of row r at
// ((c >> kb_shift) * rows + r) * kb + c % kb, kb = 1 << kb_shift, so that
// each kb-column block of all rows is one contiguous [rows][kb] slab.
struct EpiGelu {
  uint16_t* C;
  int64_t ldc;
  int rows;
  int kb_shift;
  __device__ uint16_t* at(int row, int col0) const {
    if (!kb_shift) return C + (int64_t)row * ldc + col0;
    const int kb = 1 << kb_shift;
    return C + ((int64_t)(col0 >> kb_shift) * rows + row) * kb + (col0 & (kb - 1));
  }
  __device__ void store4(int row, int col0, const float* v) const {
    float g[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) g[r] = gelu_erf_bf16(v[r]);
    *reinterpret_cast<uint2*>(at(row, col0)) = uint2{pack_bf16(g[0], g[1]), pack_bf16(g[2], g[3])};
  }
  __device__ void store8(int row, int col0, const float* v) const {
    float g[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) g[r] = gelu_erf_bf16(v[r]);
    *reinterpret_cast<u32x4*>(at(row, col0)) =
        u32x4{pack_bf16(g[0], g[1]), pack_bf16(g[2], g[3]), pack_bf16(g[4], g[5]),
              pack_bf16(g[6], g[7])};
  }
};

// GeLU(acc) kept in fp32 (the fp32 products), row stride ldc.
struct EpiGeluF32 {
  float* C;
  int64_t ldc;
  __device__ void store4(int row, int col0, const float* v) const {
    float g[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) g[r] = gelu_erf(v[r]);
    store_run4(C, ldc, OUT_F32, row, col0, g);
  }
  __device__ void store8(int row, int col0, const float* v) const {
    float g[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) g[r] = gelu_erf(v[r]);
    store_run8(C, ldc, OUT_F32, row, col0, g);
  }
};

// out = S + acc: the product added to an fp32 matrix S (the pre-summed
// other operands of a fused reduce), rounded once to the output type.
struct EpiAdd {
  const float* S;
  void* out;
  int64_t ld;  // row stride of S and out
  int odt;     // OutType
  __device__ void store4(int row, int col0, const float* v) const {
    const f32x4 x = __builtin_nontemporal_load(
        reinterpret_cast<const f32x4*>(S + (int64_t)row * ld + col0));
    float s[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = x[e] + v[e];
    store_run4(out, ld, odt, row, col0, s);
  }
  __device__ void store8(int row, int col0, const float* v) const {
    const f32x4* q = reinterpret_cast<const f32x4*>(S + (int64_t)row * ld + col0);
    const f32x4 x0 = __builtin_nontemporal_load(q), x1 = __builtin_nontemporal_load(q + 1);
    float s[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[e] = x0[e] + v[e];
      s[4 + e] = x1[e] + v[4 + e];
    }
    store_run8(out, ld, odt, row, col0, s);
  }
  // RB rows of 8 columns (col0 < N): the loads of all rows are issued before
  // any add, so 2*RB loads per lane are in flight; rows >= M read a clamped
  // row and are not stored.
  template <int RB>
  __device__ void store8_rows(const int* row, int M, int col0, float (*v)[8]) const {
    f32x4 x[RB][2];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const f32x4* q =
          reinterpret_cast<const f32x4*>(S + (int64_t)min(row[b], M - 1) * ld + col0);
      x[b][0] = __builtin_nontemporal_load(q);
      x[b][1] = __builtin_nontemporal_load(q + 1);
    }
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      float s[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[e] = x[b][0][e] + v[b][e];
        s[4 + e] = x[b][1][e] + v[b][4 + e];
      }
      if (row[b] < M) store_run8(out, ld, odt, row[b], col0, s);
    }
  }
};

// fp32 partial product of one K part (a split K): part p's [M, ncols]
// block of P at p * part_stride, columns counted from c_base.
struct EpiPart {
  float* P;
  int64_t ldp;
  int64_t part_stride;
  int c_base;
  int part;
  __device__ void store4(int row, int col0, const float* v) const {
    store_run4(P + part * part_stride, ldp, OUT_F32, row, col0 - c_base, v);
  }
  __device__ void store8(int row, int col0, const float* v) const {
    store_run8(P + part * part_stride, ldp, OUT_F32, row, col0 - c_base, v);
  }
};

// Epilogues that are told which K part they store.
template <class Epi>
struct PerPart {
  static constexpr bool value = false;
};
template <>
struct PerPart<EpiPart> {
  static constexpr bool value = true;
};

// Rows per epilogue call in the GEMM's store loop (see the kernel).
template <class Epi>
struct RowBatch {
  static constexpr int value = 1;
};
template <>
struct RowBatch<EpiAdd> {
  static constexpr int value = 4;
};

// Scatter of the QKV projection into the attention workspace (d == 128).
struct EpiQkv {
  QkvOut q;
  __device__ void store8(int row, int col0, const float* v) const {
    store4(row, col0, v);
    store4(row, col0 + 4, v + 4);
  }
  __device__ void store4(int row, int col0, const float* v) const {
    const int hall = col0 >> 7;          // head index over [Q | K | V]
    const int dd = col0 & 127;
    const int sec = hall / q.nl;         // 0 = Q, 1 = K, 2 = V
    const int head = hall - sec * q.nl;
    const int b = row / q.seq;
    const int s = row - b * q.seq;
    const int64_t bh = (int64_t)b * q.nl + head;
    if (sec < 2) {
      // Q, K: fp16, rounded to nearest even
      uint32_t w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = __builtin_bit_cast(uint16_t, (_Float16)v[r]);
      const int64_t off = (bh * q.seq_pad + s) * 128 + dd;
      *reinterpret_cast<uint2*>((sec == 0 ? q.q : q.k) + off) =
          uint2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
    } else {
      // V: fp16 hi/lo pair (the probabilities multiplying it are fp16)
      const int64_t off = (bh * 128 + dd) * q.seq_pad + s;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const _Float16 vh = (_Float16)v[r];
        const _Float16 vl = (_Float16)(v[r] - (float)vh);
        q.vt_hi[off + (int64_t)r * q.seq_pad] = __builtin_bit_cast(uint16_t, vh);
        q.vt_lo[off + (int64_t)r * q.seq_pad] = __builtin_bit_cast(uint16_t, vl);
      }
    }
  }
  // V^T written down the columns: true when the 64 columns at c0 are all V
  // and 8-token groups never cross a sequence (seq a multiple of 8), so
  // store_col8 can write 8 consecutive tokens of one head dim as one
  // 16-byte vector (wave-uniform).
  __device__ bool column_tile(int c0) const {
    return (q.seq & 7) == 0 && (c0 >> 7) >= 2 * q.nl;
  }
  // Rows row..row+7 (tokens; row a multiple of 8) of V column col.
  __device__ void store_col8(int row, int col, int M, const float* v) const {
    const int dd = col & 127;
    const int head = (col >> 7) - 2 * q.nl;
    const int b = row / q.seq;
    const int s = row - b * q.seq;
    const int64_t off = (((int64_t)b * q.nl + head) * 128 + dd) * q.seq_pad + s;
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const _Float16 vh = (_Float16)v[r];
      const _Float16 vl = (_Float16)(v[r] - (float)vh);
      hi[r] = __builtin_bit_cast(uint16_t, vh);
      lo[r] = __builtin_bit_cast(uint16_t, vl);
    }
    if (row + 8 <= M) {
      *reinterpret_cast<u32x4*>(q.vt_hi + off) =
          u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)};
      *reinterpret_cast<u32x4*>(q.vt_lo + off) =
          u32x4{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)};
    } else {
      for (int r = 0; r < 8 && row + r < M; ++r) {
        q.vt_hi[off + r] = (uint16_t)hi[r];
        q.vt_lo[off + r] = (uint16_t)lo[r];
      }
    }
  }
};

// Epilogues that can write some tiles down the columns (column_tile,
// store_col8) instead of along the rows.
template <class E>
struct ColumnRuns {
  static constexpr bool value = false;
};
template <>
struct ColumnRuns<EpiQkv> {
  static constexpr bool value = true;
};

// Tile index with the XCD-contiguous remap and grouped (8 tile-rows) order.
// With a K split the grid holds `parts` copies of the tile grid, part p
// (the K columns [p*kpart, (p+1)*kpart)) at linear ids [p*tiles, (p+1)*tiles),
// so each XCD's run covers whole groups of one part.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm,
                                            int& tn, int& part) {
  const int bid = blockIdx.x;
  const int nb = gridDim.x;
  const int xcd = bid & 7, j = bid >> 3, q = nb >> 3, r = nb & 7;
  int lin = xcd * q + (xcd < r ? xcd : r) + j;
  part = lin / (tiles_m * tiles_n);
  lin -= part * (tiles_m * tiles_n);
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int g = lin / per_group;
  const int first_m = g * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int w = lin - g * per_group;
  tm = first_m + w % gsize;
  tn = w / gsize;
}

__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  int part;
  tile_coords(tiles_m, tiles_n, tm, tn, part);
}

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------
constexpr int BUF_FLAGS = 0x00020000;  // raw buffer, 32-bit data format
constexpr int OOB = 0x7FFFFFF0;        // offset past any buffer: reads return 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > (int64_t)OOB ? OOB : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, BUF_FLAGS);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Global -> LDS copy of 16 bytes per lane (buffer_load ... lds): lane l's
// bytes land at LDS address lds_base + 16*l.  Issued from inline assembly so
// the compiler does not treat later LDS reads as waiting on it; completion is
// tracked explicitly with wait_vmcnt().  (m0 is set here and used by nothing
// else in the kernels of this file.)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, int voffset,
                                      uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_lgkmcnt0() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Workgroup barrier that is also a compiler memory barrier but adds no wait.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int N>
struct IC {
  static constexpr int value = N;
};

// f(IC<I>{}), f(IC<I+1>{}), ..., f(IC<E-1>{}), unrolled at compile time.
template <int I, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(IC<I>{});
    static_for<I + 1, E>(f);
  }
}


// Epilogue through LDS: per 32-row slab, each wave parks its fp32
// accumulators in its own LDS region (32 x WCOLS, padded) and reads them back
// as runs of 8 consecutive columns for 16-byte stores.  A wave only touches
// its own region and LDS operations of one wave complete in order, so no
// barrier is needed between the slabs.  (r0, c0) is the wave's first output
// row and column; the caller has drained every DMA into the LDS and met the
// other waves at a barrier.
// 32x32 accumulator layout: lane l, register e holds row
// 8*(e/4) + 4*(l/32) + e%4 and column l%32 of the block.
template <int WCOLS, int FM, int FN, class Epi>
__device__ __forceinline__ void epilogue_lds(uint8_t* smem, f32x16 (&acc)[FM][FN],
                                             const Epi& epi, int M, int N, int r0,
                                             int c0, int wave, int lane) {
  static_assert(WCOLS == FN * 32, "wave tile width");
  constexpr int PITCH = WCOLS + 4;
  float* stage_f = reinterpret_cast<float*>(smem) + wave * 32 * PITCH;
  constexpr int RUNS = WCOLS / 8;                 // 8-column runs per row
  constexpr int PASSES = 32 * RUNS / 64;          // wave passes per slab
  static_assert(PASSES * 64 == 32 * RUNS, "runs tile the slab");
  // An epilogue that reads memory takes RB passes per call so that the
  // loads of several rows are in flight together.
  // The passes of one call share a column only when 64 is a multiple of
  // the runs per row.
  constexpr int RB0 = RowBatch<Epi>::value;
  constexpr int RB = (64 % RUNS == 0 && PASSES % RB0 == 0) ? RB0 : 1;
#pragma unroll
  for (int mi = 0; mi < FM; ++mi) {
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int i = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        stage_f[i * PITCH + ni * 32 + (lane & 31)] = acc[mi][ni][e];
      }
    asm volatile("" ::: "memory");  // keep the LDS writes before the reads
    bool rows_left = true;
    if constexpr (ColumnRuns<Epi>::value) {
      // 32-column groups the epilogue writes down the columns: lane l takes
      // column l%32 and, per store, 8 rows, the two lane halves adjacent
      // 8-row runs (16 rows per store, 32 per group).
      rows_left = false;
#pragma unroll
      for (int ni = 0; ni < FN; ++ni) {
        const int cg = c0 + ni * 32;
        if (!epi.column_tile(cg)) {
          rows_left = true;
          continue;
        }
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int rr = 16 * g + 8 * (lane >> 5);
          const int row = r0 + mi * 32 + rr;
          float v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = stage_f[(rr + i) * PITCH + ni * 32 + (lane & 31)];
          if (row < M && cg + (lane & 31) < N) epi.store_col8(row, cg + (lane & 31), M, v);
        }
      }
    }
    if (rows_left) {
#pragma unroll 1
      for (int it = 0; it < PASSES; it += RB) {
        float v[RB][8];
        int row[RB], col0[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const int q = (it + b) * 64 + lane;
          const int rr = q / RUNS, c8 = (q % RUNS) * 8;
          row[b] = r0 + mi * 32 + rr;
          col0[b] = c0 + c8;
          const f32x4 va = *reinterpret_cast<const f32x4*>(stage_f + rr * PITCH + c8);
          const f32x4 vb = *reinterpret_cast<const f32x4*>(stage_f + rr * PITCH + c8 + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[b][e] = va[e];
            v[b][4 + e] = vb[e];
          }
        }
        if constexpr (RB == 1) {
          // (groups written down the columns above are skipped; c0 is a
          // multiple of 32, so a run's group starts at col0 & ~31)
          bool done = false;
          if constexpr (ColumnRuns<Epi>::value) done = epi.column_tile(col0[0] & ~31);
          if (row[0] < M && col0[0] < N && !done) epi.store8(row[0], col0[0], v[0]);
        } else {
          static_assert(!ColumnRuns<Epi>::value, "row batches write every run");
          if (col0[0] < N) epi.template store8_rows<RB>(row, M, col0[0], v);
        }
      }
    }
    asm volatile("" ::: "memory");  // and this slab's reads before the next writes
  }
}

// KS MFMA k-steps of 16 per pipeline stage (stage K = BK = 16 KS) and an LDS
// ring of NSL stages.  KS = 2 gives 64-byte A rows per stage; KS = 4 gives
// 128-byte A rows (a whole cache line per row per DMA), at the price of
// fewer, larger ring slots.  NA = 2 (mixed precision, KS = 2, NSL = 4):
// C = A_hi fp16(B) + A_lo bf8(B), A_hi fp16 K-blocked by 32,
// [K/32][lda][32], then A_lo bf8 K-blocked by 64, [K/64][lda][64 bytes],
// each 64-byte row piece permuted so that byte 32h + 8s + j holds column
// 16s + 8h + j (K a multiple of 64).  B stays bf16 in LDS; each k-step's B
// fragments are converted in registers to fp16 (exact for bf16 values of
// magnitude 2^-14 .. 65504) for the hi product and to bf8 for the lo
// product.  Every step brings A_hi's and B's stage; odd steps also bring
// A_lo for two stages into one of two lo slots, and at the end of the
// second stage of each pair the lo product runs as 32x32x64 bf8 MFMAs (half
// the matrix-pipe time of the fp16 pass), its B fragments gathered from the
// pair's four k-steps (lane l holds column l%32 with, for k-step s, columns
// 16s + 8(l/32) + 0..7, which is why A_lo's row pieces are permuted to
// match).
// AP (A pairs; KS = 2, row-major A, NSL = 4): A goes into two slots of
// 128-byte rows, each holding the K columns of two consecutive stages, so
// every A DMA reads whole 128-byte lines of A's rows (a stage's 64-byte row
// pieces would cost a half-used line each); B keeps its ring of NSL
// stages.  Even steps load the A pair of the stages two and three ahead
// with their B, odd steps B alone.
template <int BM, int BN, int WM, int WN, int KS, int NSL, class Epi, bool AKB, int NA = 1,
          bool AP = false>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_bf16_kernel(const uint16_t* __restrict__ A, int64_t lda,
                 const uint16_t* __restrict__ B, int64_t ldb, int M, int N,
                 int K, int tiles_m, int tiles_n, int n_base, int kpart, Epi epi) {
  // With AKB, A is K-blocked by the stage depth BK: [ceil(K/BK)][lda][BK],
  // lda the padded row count, so a stage's A tile is one contiguous run of
  // rows.  The grid covers output columns [n_base, N) (tiles_n tiles wide);
  // all coordinates are absolute.  A grid of several copies of the tile grid
  // splits K: copy p multiplies K columns [p*kpart, min((p+1)*kpart, K))
  // (kpart a multiple of BK, every part non-empty) and hands its partial
  // product to an epilogue that stores per part.
  static_assert(KS == 2 || KS == 4, "k-steps per stage");
  static_assert(NSL >= 3 && NSL <= 6, "ring slots");
  static_assert(NA == 1 || (NA == 2 && AKB && KS == 2 && NSL == 4), "mixed A: the layout below");
  constexpr bool MIX = NA == 2;
  constexpr int NAO = MIX ? 1 : NA;  // A operands in the stage ring
  static_assert(!AP || (KS == 2 && !AKB && NA == 1 && NSL == 4), "A pairs: the layout below");
  constexpr int BK = 16 * KS;
  constexpr int NW = WM * WN;
  constexpr int FM = BM / WM / 32;
  constexpr int FN = BN / WN / 32;
  constexpr int A_ROWB = AP ? 128 : BK * 2;  // A rows in LDS: 64 or 128 bytes
  constexpr int CPR = A_ROWB / 16;         // 16-byte chunks per A row (4 or 8)
  constexpr int RPD = 64 / CPR;            // A rows per 1 KiB DMA
  constexpr int ASH = CPR == 4 ? 2 : 1;    // A swizzle: chunk ^ ((row >> ASH) & (CPR-1))
  constexpr int B_ROWB = BN * 2;           // B rows in LDS: natural [k][n]
  constexpr int B_CH = B_ROWB / 16;        // 16-byte chunks per B row
  constexpr int A_STAGE = BM * A_ROWB;        // one A slot (AP: a pair of stages)
  constexpr int B_STAGE = BK * B_ROWB;
  constexpr int A_DMA = A_STAGE / 1024 / NW;  // 1 KiB DMAs per wave per A slot
  constexpr int B_DMA = B_STAGE / 1024 / NW;
  constexpr int NDMA = NAO * A_DMA + B_DMA;    // AP: even steps; odd steps B_DMA
  constexpr int A_SLOTS = AP ? 2 : NSL;
  constexpr int LO_STAGE = MIX ? BM * 64 : 0;  // MIX: A_lo of two stages (bf8)
  constexpr int LO_DMA = LO_STAGE / 1024 / NW;  // MIX: on odd steps
  static_assert(A_DMA * 1024 * NW == A_STAGE && B_DMA * 1024 * NW == B_STAGE, "DMA split");
  static_assert(B_CH % 16 == 0 || B_CH == 24, "B swizzle: 256-byte multiple or 384-byte rows");
  static_assert(FM >= 1 && FN >= 1, "wave tile");

  // LDS ring: slot s holds A operand o at (s*NAO + o)*A_STAGE (AP: pair slot
  // s at s*A_STAGE) and B at A_SLOTS*NAO*A_STAGE + s*B_STAGE; MIX: the two
  // lo slots follow.  The same memory later stages the epilogue (NW regions
  // of 32 x (BN/WN+4)).
  constexpr int PIPE_BYTES = A_SLOTS * NAO * A_STAGE + NSL * B_STAGE + 2 * LO_STAGE;
  constexpr int EPI_BYTES = NW * 32 * (BN / WN + 4) * 4;
  __shared__ __attribute__((aligned(16))) uint8_t
      smem[PIPE_BYTES > EPI_BYTES ? PIPE_BYTES : EPI_BYTES];
  uint8_t* const lds_a = smem;
  uint8_t* const lds_b = smem + A_SLOTS * NAO * A_STAGE;
  uint8_t* const lds_lo = lds_b + NSL * B_STAGE;
  const uint32_t lds_a_addr = (uint32_t)(uintptr_t)(lds_u8*)lds_a;
  const uint32_t lds_b_addr = (uint32_t)(uintptr_t)(lds_u8*)lds_b;
  const uint32_t lds_lo_addr = (uint32_t)(uintptr_t)(lds_u8*)lds_lo;

  int tm, tn, part;
  tile_coords(tiles_m, tiles_n, tm, tn, part);
  if constexpr (NA == 1) {  // (paired A operands are never split)
    if (part > 0) {  // this part's K columns: shift A and B, shorten K
      const int kbeg = part * kpart;
      A += AKB ? (int64_t)(kbeg / BK) * lda * BK : (int64_t)kbeg;
      B += (int64_t)kbeg * ldb;
      K -= kbeg;
    }
  }
  if (K > kpart) K = kpart;
  const int m0 = tm * BM, n0 = n_base + tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr0 = (wave / WN) * (BM / WM);
  const int wc0 = (wave % WN) * (BN / WN);
  const int rows_valid = min(BM, M - m0);
  const int cols_valid = min(BN, N - n0);

  // ---- DMA lane offsets.  A: RPD rows of A_ROWB bytes per DMA; lane l
  // fills row l/CPR, physical chunk l%CPR with logical chunk
  // (l%CPR) ^ ((row >> ASH) & (CPR-1)).  B: the DMAs fill the packed rows
  // in order, 16-byte chunk q = 64*(DMA index) + l landing in row q/B_CH,
  // slot q%B_CH, which holds logical chunk slot ^ bswz(row).  The swizzles
  // keep the fragment reads on distinct banks (any 16 consecutive A rows at
  // one logical chunk cover 16 distinct 16-byte bank groups; the four B rows
  // of one transposed read land in four distinct 64-byte bank ranges); they
  // are applied to the global addresses.
  int a_off[A_DMA], a_col[A_DMA];
#pragma unroll
  for (int j = 0; j < A_DMA; ++j) {
    const int row = RPD * (j * NW + wave) + lane / CPR;
    const int c = (lane % CPR) ^ ((row >> ASH) & (CPR - 1));
    a_off[j] = AKB ? row * A_ROWB + c * 16 : row * (int)lda * 2 + c * 16;
    a_col[j] = c * 8;
  }
  // B rows a multiple of 256 bytes apart start on the same bank, so the
  // rows of a read are spread by 64-byte blocks; 384-byte rows alternate
  // between two bank halves, so only row bit 1 selects the block.
  auto bswz = [](int row) { return B_CH == 24 ? ((row >> 1) & 1) << 2 : (row & 3) << 2; };
  int b_off[B_DMA];
#pragma unroll
  for (int j = 0; j < B_DMA; ++j) {
    const int q = (j * NW + wave) * 64 + lane;
    const int row = q / B_CH;
    const int c = (q % B_CH) ^ bswz(row);
    b_off[j] = row * (int)ldb * 2 + c * 16;
  }

  // K blocks of each A operand (A_2's blocks start after A_1's)
  const int a_blocks = (K + BK - 1) / BK;
  // AP: the A DMA number ja (0 <= ja < A_DMA) of pair p (K columns 64p ..
  // 64p+63) into pair slot PS.
  auto dma_a_pair = [&](int p, auto PS, int ja) {
    constexpr int ps = decltype(PS)::value;
    const int k0 = p * 2 * BK;
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(A + (int64_t)m0 * lda + k0, (int64_t)rows_valid * lda * 2 - (int64_t)k0 * 2);
    const int off = (k0 + a_col[ja] < K) ? a_off[ja] : OOB;
    dma16(ra, off, lds_a_addr + ps * A_STAGE + (ja * NW + wave) * 1024);
  };
  // DMA number j (0 <= j < NDMA) of stage kt into ring slot SLOT.
  auto dma = [&](int kt, auto SLOT, int j) {
    constexpr int slot = decltype(SLOT)::value;
    const int k0 = kt * BK;
    if (j < NAO * A_DMA) {
      const int op = j / A_DMA, ja = j - op * A_DMA;
      const int blk = kt + op * a_blocks;
      const __amdgpu_buffer_rsrc_t ra =
          AKB ? make_rsrc(A + ((int64_t)blk * lda + m0) * BK, (int64_t)rows_valid * A_ROWB)
              : make_rsrc(A + (int64_t)m0 * lda + k0, (int64_t)rows_valid * lda * 2 - (int64_t)k0 * 2);
      const int off = (k0 + a_col[ja] < K) ? a_off[ja] : OOB;
      dma16(ra, off, lds_a_addr + (slot * NAO + op) * A_STAGE + (ja * NW + wave) * 1024);
    } else {
      const int jb = j - NAO * A_DMA;
      const __amdgpu_buffer_rsrc_t rb =
          make_rsrc(B + (int64_t)k0 * ldb + n0,
                    ((int64_t)(K - k0) - 1) * ldb * 2 + (int64_t)cols_valid * 2);
      dma16(rb, b_off[jb], lds_b_addr + slot * B_STAGE + (jb * NW + wave) * 1024);
    }
  };
  // MIX: DMA number ja (0 <= ja < LO_DMA) of A_lo pair p (K columns 64p ..
  // 64p+63, 64-byte rows like A_hi's, same offsets and swizzle) into lo
  // slot LS.
  auto dma_lo = [&](int p, auto LS, int ja) {
    constexpr int ls = decltype(LS)::value;
    const uint8_t* const a_lo =
        reinterpret_cast<const uint8_t*>(A) + (int64_t)a_blocks * lda * 64;
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(a_lo + ((int64_t)p * lda + m0) * 64, (int64_t)rows_valid * 64);
    const int off = (p * 64 < K) ? a_off[ja] : OOB;
    dma16(ra, off, lds_lo_addr + ls * LO_STAGE + (ja * NW + wave) * 1024);
  };

  // ---- fragment read addresses (byte offsets inside a slot).
  // A (ds_read_b128): row wr0 + mi*32 + (lane&31), chunk 2ks + (lane>>5)
  // (AP: of half h of the pair slot, chunk 2(h KS + ks) + (lane>>5)).
  constexpr int AH = AP ? 2 : 1;
  int a_rd[AH][KS];
#pragma unroll
  for (int h = 0; h < AH; ++h)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = (2 * (h * KS + ks) + (lane >> 5)) ^ (((lane & 31) >> ASH) & (CPR - 1));
      a_rd[h][ks] = (wr0 + (lane & 31)) * A_ROWB + c * 16;
    }
  // B (ds_read_b64_tr_b16): in each 16-lane group G, input lane r points at
  // row 8*(G>>1) + r/4 and columns 16*(G&1) + 4*(r&3) of the wave's 32-column
  // block; the transposed read leaves lane l holding column l%32 with
  // k = 8*(l/32) + 0..3; a second read 4 rows down gives k + 4..7.
  int b_rd[FN];
  {
    const int G = lane >> 4, r = lane & 15;
    const int krow = 8 * (G >> 1) + (r >> 2);
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
      // (the rows read, krow + 4 and + 16*ks, all have krow's low two bits)
      const int c = (((wc0 + ni * 32) >> 3) + 2 * (G & 1) + ((r & 3) >> 1)) ^ bswz(krow);
      b_rd[ni] = krow * B_ROWB + c * 16 + (r & 1) * 8;
    }
  }

  f32x16 acc[FM][FN];
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.0f;

  bf16x8 fa[2][NAO][FM], fb[2][FN];
  // Fragment read unit q of k-step ks from ring slot SLOT into set fset:
  // units 0..FN-1 are B fragments (two transposed reads each), units
  // FN..FN+NA*FM-1 are A fragments (operand by operand).
  auto read_unit = [&](auto SLOT, int ks, int fset, int q) {
    constexpr int slot = decltype(SLOT)::value;
    if (q < FN) {
      const uint8_t* lb = lds_b + slot * B_STAGE + ks * 16 * B_ROWB + b_rd[q];
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)lb);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(lb + 4 * B_ROWB));
      fb[fset][q] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else if constexpr (AP) {
      // stage kt in B slot kt % 4: A pair slot (kt / 2) % 2, half kt % 2
      const int mi = q - FN;
      fa[fset][0][mi] = *reinterpret_cast<const bf16x8*>(
          lds_a + ((slot >> 1) & 1) * A_STAGE + a_rd[slot & 1][ks] + mi * 32 * A_ROWB);
    } else {
      const int op = (q - FN) / FM, mi = (q - FN) - op * FM;
      fa[fset][op][mi] = *reinterpret_cast<const bf16x8*>(
          lds_a + (slot * NAO + op) * A_STAGE + a_rd[0][ks] + mi * 32 * A_ROWB);
    }
  };
  // one MFMA of a k-step, idx in [0, NAO*FM*FN): operand by operand (NA =
  // 1 with AP or plain: one operand); MIX: the fp16 product of A_hi and the
  // converted B fragments
  auto mfma1 = [&](int fset, int idx) {
    const int op = idx / (FM * FN), r = idx - op * (FM * FN);
    const int mi = r / FN, ni = r % FN;
    if constexpr (MIX)
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
          __builtin_bit_cast(f16x8, fa[fset][op][mi]), __builtin_bit_cast(f16x8, fb[fset][ni]),
          acc[mi][ni], 0, 0, 0);
    else
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[fset][op][mi], fb[fset][ni],
                                                            acc[mi][ni], 0, 0, 0);
  };
  // MIX: B fragment ni of set fset (bf16, k-step s = 0..3 of its stage pair)
  // -> fp16 in place (round toward zero, exact for bf16 values in fp16's
  // normal range) and bf8 (nearest even) into words 2s, 2s+1 of blo[ni].
  i32x8 blo[MIX ? FN : 1];
  auto convert_b = [&](int fset, int ni, int sk) {
    const u32x4 d = __builtin_bit_cast(u32x4, fb[fset][ni]);
    float lo[4], hi[4];
    u32x4 h;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      lo[w] = __uint_as_float(d[w] << 16);
      hi[w] = __uint_as_float(d[w] & 0xffff0000u);
      h[w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo[w], hi[w]));
    }
    fb[fset][ni] = __builtin_bit_cast(bf16x8, h);
    blo[ni][2 * sk] = __builtin_amdgcn_cvt_pk_bf8_f32(
        lo[1], hi[1], __builtin_amdgcn_cvt_pk_bf8_f32(lo[0], hi[0], 0, false), true);
    blo[ni][2 * sk + 1] = __builtin_amdgcn_cvt_pk_bf8_f32(
        lo[3], hi[3], __builtin_amdgcn_cvt_pk_bf8_f32(lo[2], hi[2], 0, false), true);
  };
  // MIX: A_lo fragment reads (row wr0 + mi*32 + lane%32, logical 16-byte
  // chunks 2(lane/32) and 2(lane/32)+1 of the 64-byte row, A's swizzle) and
  // the lo product, bf8 x bf8 with unit scales (E8M0 127).
  i32x8 alo[MIX ? FM : 1];
  auto read_lo = [&](auto LS, int mi) {
    constexpr int ls = decltype(LS)::value;
    const uint8_t* base =
        lds_lo + ls * LO_STAGE + mi * 32 * A_ROWB + (wr0 + (lane & 31)) * A_ROWB;
    const int sw = ((lane & 31) >> ASH) & (CPR - 1);
    const u32x4 x0 = *reinterpret_cast<const u32x4*>(base + ((2 * (lane >> 5)) ^ sw) * 16);
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(base + ((2 * (lane >> 5) + 1) ^ sw) * 16);
    alo[mi] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                    (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  };
  auto mfma_lo = [&](int idx) {
    const int mi = idx / FN, ni = idx % FN;
    acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(alo[mi], blo[ni], acc[mi][ni],
                                                                  1, 1, 0, 127, 0, 127);
  };

  // Stages past the end of K load zeros (offsets outside the buffers), so
  // every step issues the same DMAs and the explicit vmcnt counts below are
  // exact.
  const int nk = (K + BK - 1) / BK;

  // One pipeline step computes stage kt from ring slot u = kt % NSL.  Each
  // MFMA is followed by at most one DMA and one fragment read unit, pinned
  // with scheduling barriers (a wave cannot issue past an MFMA until the
  // matrix pipe accepts it, so traffic must sit between MFMAs to overlap):
  //   k-steps 0..KS-2: at their start the fragment reads of the next
  //     k-step; the DMAs of stage kt+NSL-1 (slot (u+NSL-1)%NSL, last read in
  //     step kt-1 before its barrier) at the end of k-step 0 (KS = 2) or
  //     spread over these k-steps (KS = 4);
  //   wait until stage kt+1's DMAs have landed (NSL-2 later stages stay in
  //   flight) and until this wave's own LDS reads are complete, so that
  //   after the barrier no read of a slot about to be refilled is pending;
  //   barrier;
  //   k-step KS-1: the fragment reads of k-step 0 of stage kt+1.
  // Fragment register sets alternate with the k-step's parity (KS even).
  constexpr int NMF = NAO * FM * FN;  // MFMAs per k-step (MIX: the fp16 ones)
  constexpr int NRU = NAO * FM + FN;  // fragment read units per k-step
  constexpr int DSLOTS = (KS - 1) * NMF;
  static_assert(NDMA + LO_DMA <= DSLOTS && NRU <= NMF, "traffic fits between the MFMAs");
  static_assert(!MIX || FM <= NMF, "MIX: A_lo reads fit between the MFMAs");
  // AP: step kt (kt % 4 == u) issues, on even u, the A pair kt/2 + 1 (the
  // stages two and three ahead) into pair slot (kt/2 + 1) % 2, then B of
  // stage kt+3; on odd u, B alone.  Stage kt+1 then needs the B issued three
  // steps back and the A pair issued at the last even step, so the loads
  // that may stay in flight are those of step kt-1 after its A pair (B) and
  // of step kt (odd u), or those after step kt-2's B (even u).
  // MIX (NSL = 4, so u's parity is kt's): odd step kt issues, after its
  // stage's DMAs, A_lo pair (kt+1)/2 into lo slot ((kt+1)/2) % 2 (that slot's
  // previous pair was read in step kt-2, before step kt-1's barrier), and
  // ends with the lo product of pair (kt-1)/2, issued at step kt-2 and so
  // landed at this step's wait; the B fragments of the pair's four k-steps
  // are converted as each k-step begins.  Steps kt-1 and kt hold one odd
  // step between them, so the loads that may stay in flight at the wait are
  // 2 NDMA + LO_DMA.
  auto step = [&](int kt, auto U) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    constexpr int nxt = (u + NSL - 1) % NSL;
    constexpr int nd = AP ? ((u & 1) ? B_DMA : A_DMA + B_DMA)
                          : NDMA + ((MIX && (u & 1)) ? LO_DMA : 0);  // DMAs this step
    // MFMA slot after which DMA d of the step is issued
    auto dma_slot = [](int d) { return KS == 2 ? NMF - nd + d : d * DSLOTS / nd; };
#pragma unroll
    for (int ksi = 0; ksi < KS - 1; ++ksi) {
#pragma unroll
      for (int j = 0; j < NMF; ++j) {
        if constexpr (MIX) {
          if (j < FN) convert_b(ksi & 1, j, 2 * (u & 1) + ksi);
        }
        mfma1(ksi & 1, j);
        __builtin_amdgcn_sched_barrier(0);
        if (j < NRU) read_unit(IC<u>{}, ksi + 1, (ksi + 1) & 1, j);
#pragma unroll
        for (int d = 0; d < nd; ++d)
          if (dma_slot(d) == ksi * NMF + j) {
            if constexpr (AP) {
              if (!(u & 1) && d < A_DMA)
                dma_a_pair(kt / 2 + 1, IC<((u >> 1) + 1) & 1>{}, d);
              else
                dma(kt + NSL - 1, IC<nxt>{}, NA * A_DMA + d - ((u & 1) ? 0 : A_DMA));
            } else if (MIX && d >= NDMA) {
              dma_lo((kt + 1) / 2, IC<((u + 1) / 2) & 1>{}, d - NDMA);
            } else {
              dma(kt + NSL - 1, IC<nxt>{}, d);
            }
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (AP)
      wait_vmcnt<(u & 1) ? 2 * B_DMA : A_DMA + 2 * B_DMA>();
    else
      wait_vmcnt<(NSL - 2) * NDMA + LO_DMA>();
    wait_lgkmcnt0();
    stage_barrier();
#pragma unroll
    for (int j = 0; j < NMF; ++j) {
      if constexpr (MIX) {
        if (j < FN) convert_b((KS - 1) & 1, j, 2 * (u & 1) + KS - 1);
      }
      mfma1((KS - 1) & 1, j);
      __builtin_amdgcn_sched_barrier(0);
      if (j < NRU) read_unit(IC<(u + 1) % NSL>{}, 0, 0, j);
      if constexpr (MIX && (u & 1)) {
        if (j < FM) read_lo(IC<((u - 1) / 2) & 1>{}, j);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MIX && (u & 1)) {
#pragma unroll
      for (int j = 0; j < FM * FN; ++j) mfma_lo(j);
    }
  };

  // Prologue: stages 0..NSL-2 in flight (MIX: then A_lo pair 0, as step -1
  // would), wait for stage 0.  AP: the loads
  // steps -3, -2, -1 would have issued (B of stage 0; A pair 0 and B of
  // stage 1; B of stage 2), then wait for A pair 0 and B of stage 0.
  if constexpr (AP) {
#pragma unroll
    for (int j = 0; j < B_DMA; ++j) dma(0, IC<0>{}, NA * A_DMA + j);
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) dma_a_pair(0, IC<0>{}, j);
#pragma unroll
    for (int j = 0; j < B_DMA; ++j) dma(1, IC<1>{}, NA * A_DMA + j);
#pragma unroll
    for (int j = 0; j < B_DMA; ++j) dma(2, IC<2>{}, NA * A_DMA + j);
    wait_vmcnt<2 * B_DMA>();
  } else {
    static_for<0, NSL - 1>([&](auto S) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < NDMA; ++j) dma(decltype(S)::value, S, j);
    });
    if constexpr (MIX) {  // step -1's lo pair
#pragma unroll
      for (int j = 0; j < LO_DMA; ++j) dma_lo(0, IC<0>{}, j);
    }
    wait_vmcnt<(NSL - 2) * NDMA + LO_DMA>();
  }
  stage_barrier();
#pragma unroll
  for (int q = 0; q < NRU; ++q) read_unit(IC<0>{}, 0, 0, q);
  int kt = 0;
  for (; kt + NSL <= nk; kt += NSL)
    static_for<0, NSL>([&](auto U) __attribute__((always_inline)) { step(kt + decltype(U)::value, U); });
  const int rem = nk - kt;  // 0..NSL-1, uniform; these steps' DMAs read zeros
  static_for<0, NSL - 1>([&](auto U) __attribute__((always_inline)) {
    if (rem > decltype(U)::value) step(kt + decltype(U)::value, U);
  });
  wait_vmcnt<0>();
  __syncthreads();

  Epi e = epi;
  if constexpr (PerPart<Epi>::value) e.part = part;
  epilogue_lds<BN / WN>(smem, acc, e, M, N, m0 + wr0, n0 + wc0, wave, lane);
}

// Tile kinds of the plain products: rows, columns, stage depth (the K
// block of a K-blocked A) and a relative efficiency per output element (the
// larger tiles are cheaper: less LDS and L2 traffic per MFMA).
struct TileKind {
  int bm, bn, bk;
  double eff;
};
constexpr int NKIND = 5;
constexpr TileKind kKinds[NKIND] = {{256, 256, 32, 1.0},
                                    {256, 192, 32, 0.95},
                                    {256, 128, 64, 0.95},
                                    {128, 192, 64, 0.80},
                                    {128, 128, 64, 0.70}};

// How an [M, N] output is covered: columns [0, n1) by tiles of kind k1,
// columns [n1, N) by tiles of kind k2 (k2 < 0: kind k1 covers all of N).
// parts > 1: the k2 rectangle splits K into parts of kpart columns, each
// part's product stored as an fp32 partial and the partials summed after.
struct Plan {
  int k1, k2, n1;
  int parts = 1, kpart = 0;
};

// Estimated time of `tiles` tiles of kind k: full waves over the compute
// units times the tile's cost.
double kind_cost(int k, int64_t tiles, int64_t ncu) {
  return (double)((tiles + ncu - 1) / ncu) * kKinds[k].bm * kKinds[k].bn / kKinds[k].eff;
}

// The cheapest plan by that estimate.  A single kind leaves its last wave
// partly idle when the tile count is not a multiple of the CU count (2048 x
// 22528 in 256x256 tiles: 704 tiles = 2.75 waves); two rectangles avoid it:
// whole waves of kind k1 over the first columns, then the remaining columns
// in a kind whose tiles fill about one wave (there: 512 tiles of 256x256,
// then 256 tiles of 256x192).  Over a K-blocked A both kinds share the
// stage depth, so one blocking serves both (a row-major A serves any pair);
// a split plan is kept only when it is estimated at least 3% cheaper than
// the best single kind.
Plan plan_columns(int M, int N, bool a_kblocked, int64_t ncu) {
  Plan best{0, -1, N};
  double best_cost = 1e300;
  for (int k = 0; k < NKIND; ++k) {
    const TileKind& t = kKinds[k];
    const int64_t tiles = (int64_t)((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
    const double c = kind_cost(k, tiles, ncu);
    if (c < best_cost * 0.999) {
      best_cost = c;
      best = Plan{k, -1, N};
    }
  }
  const double single = best_cost;
  for (int k1 = 0; k1 < NKIND; ++k1) {
    const TileKind& t1 = kKinds[k1];
    const int64_t tm1 = (M + t1.bm - 1) / t1.bm;
    const int64_t step = ncu / std::gcd(ncu, tm1);  // tile columns per whole waves
    int64_t cols1 = (N / t1.bn) / step * step;
    if (cols1 * t1.bn >= N) cols1 -= step;
    if (cols1 <= 0) continue;
    const int n1 = (int)(cols1 * t1.bn);
    const double c1 = (double)(tm1 * cols1 / ncu) * t1.bm * t1.bn / t1.eff;
    for (int k2 = 0; k2 < NKIND; ++k2) {
      const TileKind& t2 = kKinds[k2];
      if (a_kblocked && t2.bk != t1.bk) continue;
      const int64_t tiles2 = (int64_t)((M + t2.bm - 1) / t2.bm) * ((N - n1 + t2.bn - 1) / t2.bn);
      const double c = c1 + kind_cost(k2, tiles2, ncu);
      if (c < best_cost * 0.999 && c <= 0.97 * single) {
        best_cost = c;
        best = Plan{k1, k2, n1};
      }
    }
  }
  return best;
}

// Seconds of one wave of kind-k tiles over K columns: the tile's FLOPs at
// one CU's share of the 256x256 kind's steady rate (about 1340 TFLOP/s on
// 256 CUs), plus a fixed cost per tile (first loads, epilogue).
constexpr double kCuFlops = 1340e12 / 256;
constexpr double kTileFixed = 8e-6;
// The fp32 partials of a split K are written and read back once at about
// this rate, by one more launch.
constexpr double kPartialBytesPerSec = 5.0e12;
constexpr double kSumLaunch = 4e-6;
// Largest partial buffer a split may use.
constexpr int64_t kMaxSplitBytes = (int64_t)1 << 30;

double wave_seconds(int k, int64_t K) {
  return kKinds[k].bm * (double)kKinds[k].bn * 2.0 * (double)K / kKinds[k].eff / kCuFlops +
         kTileFixed;
}

double rect_seconds(int k, int M, int cols, int64_t K, int parts, int64_t ncu) {
  if (cols <= 0) return 0.0;
  const int64_t tiles = (int64_t)((M + kKinds[k].bm - 1) / kKinds[k].bm) *
                        ((cols + kKinds[k].bn - 1) / kKinds[k].bn) * parts;
  return (double)((tiles + ncu - 1) / ncu) * wave_seconds(k, K);
}

// With a long K (k_split > 0, the row-parallel product over a K-blocked
// A), a plan may instead run whole waves of 256x256 tiles over the first
// columns and the rest (often less than a wave of tiles) as 256x256 tiles
// over 2-8 parts of K: a wave of short tiles instead of a partly idle wave
// of full-length ones, for one round trip of fp32 partials.  At 2048 rows
// and 10240 columns (320 tiles of 256x256): 256 full tiles, then 64 tiles
// in 4 parts.  Taken when its estimate is at least 3% below the plan above.
Plan plan_bf16(int M, int N, bool a_kblocked, int64_t k_split) {
  const int64_t ncu = device_cu_count();
  const Plan cols = plan_columns(M, N, a_kblocked, ncu);
  if (k_split <= 0) return cols;
  const double t_cols =
      rect_seconds(cols.k1, M, cols.n1, k_split, 1, ncu) +
      (cols.k2 >= 0 ? rect_seconds(cols.k2, M, N - cols.n1, k_split, 1, ncu) : 0.0);
  const int64_t tm = (M + 255) / 256;
  const int64_t step = ncu / std::gcd(ncu, tm);
  int64_t whole = (N / 256) / step * step;
  if (whole * 256 >= N) whole -= step;
  Plan best = cols;
  double best_t = 0.97 * t_cols;
  for (const int64_t cols1 : {whole, (int64_t)0}) {
    if (cols1 < 0) continue;
    const int n1 = (int)(cols1 * 256), rest = N - n1;
    if (rest <= 0) continue;
    for (const int want : {2, 3, 4, 6, 8}) {
      const int64_t kpart = (k_split + want * 32 - 1) / (want * 32) * 32;
      const int parts = (int)((k_split + kpart - 1) / kpart);
      if (parts < 2 || (int64_t)parts * M * rest * 4 > kMaxSplitBytes) continue;
      const double t = rect_seconds(0, M, n1, k_split, 1, ncu) +
                       rect_seconds(0, M, rest, kpart, parts, ncu) +
                       8.0 * parts * M * rest / kPartialBytesPerSec + kSumLaunch;
      if (t < best_t) {
        best_t = t;
        best = Plan{0, 0, n1, parts, (int)kpart};
      }
    }
  }
  return best;
}

template <int BM, int BN, int WM, int WN, int KS, int NSL, bool AKB, class Epi, int NA = 1,
          bool AP = false>
hipError_t launch_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M,
                       int N, int K, const Epi& epi, hipStream_t s, int n_base = 0,
                       int parts = 1, int kpart = 0) {
  const int tm = (M + BM - 1) / BM, tn = (N - n_base + BN - 1) / BN;
  if (tm <= 0 || tn <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, KS, NSL, Epi, AKB, NA, AP>),
                     dim3(tm * tn * parts), dim3(WM * WN * 64), 0, s, A, lda, B, ldb, M, N, K, tm,
                     tn, n_base, parts > 1 ? kpart : K, epi);
  return hipGetLastError();
}

// Output columns [n_base, n_end) in tiles of kind k (over `parts` parts of
// kpart K columns when parts > 1).
template <bool AKB, class Epi>
hipError_t launch_kind(int k, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                       int M, int n_base, int n_end, int K, const Epi& epi, hipStream_t s,
                       int parts = 1, int kpart = 0) {
  // K = 32 stages over a row-major A read it through A pairs (whole 128-byte
  // lines of its rows)
  switch (k) {
    case 0:
      if constexpr (AKB)
        return launch_bf16<256, 256, 2, 2, 2, 5, AKB>(A, lda, B, ldb, M, n_end, K, epi, s, n_base,
                                                      parts, kpart);
      else
        return launch_bf16<256, 256, 2, 2, 2, 4, AKB, Epi, 1, true>(A, lda, B, ldb, M, n_end, K,
                                                                   epi, s, n_base, parts, kpart);
    case 1:
      if constexpr (AKB)
        return launch_bf16<256, 192, 2, 2, 2, 5, AKB>(A, lda, B, ldb, M, n_end, K, epi, s, n_base,
                                                      parts, kpart);
      else
        return launch_bf16<256, 192, 2, 2, 2, 4, AKB, Epi, 1, true>(A, lda, B, ldb, M, n_end, K,
                                                                   epi, s, n_base, parts, kpart);
    case 2:
      return launch_bf16<256, 128, 2, 2, 4, 3, AKB>(A, lda, B, ldb, M, n_end, K, epi, s, n_base,
                                                    parts, kpart);
    case 3:
      return launch_bf16<128, 192, 2, 2, 4, 3, AKB>(A, lda, B, ldb, M, n_end, K, epi, s, n_base,
                                                    parts, kpart);
    default:
      return launch_bf16<128, 128, 2, 2, 4, 3, AKB>(A, lda, B, ldb, M, n_end, K, epi, s, n_base,
                                                    parts, kpart);
  }
}

// K block (stage depth) of the plan for an [M, N] output over K (k_split:
// K when the product may split it, else 0): 32 for 256x256 and 256x192
// tiles (five stages fill the LDS), 64 for the others.
int a_block(int M, int N, int64_t k_split) {
  return kKinds[plan_bf16(M, N, true, k_split).k1].bk;
}

// C[r, n1 + c] = S[r, n1 + c] (when S is given) + sum over the parts of
// P[p][r][c], in part order, rounded once to the output type: the sum of a
// split K.  8 columns per thread (ncols % 8 == 0), grid-stride over rows.
__global__ void __launch_bounds__(256)
splitk_sum_kernel(const float* __restrict__ P, int parts, int64_t part_stride, int ncols,
                  const float* __restrict__ S, void* C, int64_t ldc, int out, int M, int n1) {
  const int64_t groups = (int64_t)M * (ncols / 8);
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < groups;
       g += (int64_t)gridDim.x * 256) {
    const int r = (int)(g / (ncols / 8)), c = (int)(g - (int64_t)r * (ncols / 8)) * 8;
    const f32x4* p = reinterpret_cast<const f32x4*>(P + (int64_t)r * ncols + c);
    f32x4 a0 = __builtin_nontemporal_load(p), a1 = __builtin_nontemporal_load(p + 1);
    for (int q = 1; q < parts; ++q) {
      const f32x4* pq = reinterpret_cast<const f32x4*>(P + q * part_stride + (int64_t)r * ncols + c);
      const f32x4 b0 = __builtin_nontemporal_load(pq), b1 = __builtin_nontemporal_load(pq + 1);
      a0 += b0;
      a1 += b1;
    }
    float v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    if (S) {
      const f32x4* sp = reinterpret_cast<const f32x4*>(S + (int64_t)r * ldc + n1 + c);
      const f32x4 s0 = __builtin_nontemporal_load(sp), s1 = __builtin_nontemporal_load(sp + 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = s0[e] + v[e];
        v[4 + e] = s1[e] + v[4 + e];
      }
    }
    store_run8(C, ldc, out, r, n1 + c, v);
  }
}

// Bytes of fp32 partials the plan of an [M, N] product over k_split K
// columns needs (0 when it does not split K).
int64_t split_bytes(int M, int N, int64_t k_split) {
  if (M <= 0 || N <= 0 || k_split <= 0) return 0;
  const Plan p = plan_bf16(M, N, true, k_split);
  return p.parts > 1 ? (int64_t)p.parts * M * (N - p.n1) * 4 : 0;
}

// AKB: A is K-blocked by the plan's stage depth (see gemm_bf16_kernel), lda
// its row count; the caller has checked the block.  With partials (fp32,
// split_bytes(M, N, K) of them; EpiStore and EpiAdd only) the plan may split
// K; without, it does not.
template <bool AKB, class Epi>
hipError_t dispatch_bf16(const uint16_t* A, int64_t lda, const uint16_t* B,
                         int64_t ldb, int M, int N, int K, const Epi& epi, hipStream_t s,
                         float* partials = nullptr) {
  if (M == 0 || N == 0) return hipSuccess;
  // tiles are addressed with 32-bit byte offsets: 256 rows of A, 64 of B
  // (K-blocked A tiles are at most 32 KiB)
  if ((!AKB && lda >= ((int64_t)1 << 22)) || ldb >= ((int64_t)1 << 24)) return hipErrorInvalidValue;
  constexpr bool kSplittable = AKB && (std::is_same_v<Epi, EpiStore> || std::is_same_v<Epi, EpiAdd>);
  const Plan p = plan_bf16(M, N, AKB, kSplittable && partials ? K : 0);
  hipError_t e = launch_kind<AKB>(p.k1, A, lda, B, ldb, M, 0, p.n1, K, epi, s);
  if (e != hipSuccess || p.k2 < 0) return e;
  if constexpr (kSplittable) {
    if (p.parts > 1) {
      // the split rectangle is 256x256 tiles (plan_bf16)
      const int ncols = N - p.n1;
      const int64_t part_stride = (int64_t)M * ncols;
      e = launch_bf16<256, 256, 2, 2, 2, 5, AKB>(A, lda, B, ldb, M, N, K,
                                                 EpiPart{partials, ncols, part_stride, p.n1, 0},
                                                 s, p.n1, p.parts, p.kpart);
      if (e != hipSuccess) return e;
      const float* S = nullptr;
      void* C;
      int64_t ldc;
      int out;
      if constexpr (std::is_same_v<Epi, EpiStore>) {
        C = epi.C;
        ldc = epi.ldc;
        out = epi.out;
      } else {
        S = epi.S;
        C = epi.out;
        ldc = epi.ld;
        out = epi.odt;
      }
      const int64_t groups = (int64_t)M * (ncols / 8);
      const int64_t blocks = std::min<int64_t>((groups + 255) / 256, 8192);
      hipLaunchKernelGGL(splitk_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, s, partials,
                         p.parts, part_stride, ncols, S, C, ldc, out, M, p.n1);
      return hipGetLastError();
    }
  }
  return launch_kind<AKB>(p.k2, A, lda, B, ldb, M, p.n1, N, K, epi, s);
}

// X [M, K] row-major (row stride lda) -> K-blocked [ceil(K/kb)][M][kb]
// (kb = 32 or 64; zeros in the columns past K of the last block), the A
// layout whose stage tiles are contiguous runs.  A wave moves 8 rows x 64
// columns, 16 bytes per lane: it reads whole 128-byte row segments and
// writes, per kb-column block, 8 consecutive rows as one contiguous run.
__global__ void __launch_bounds__(256)
kblock_kernel(const uint16_t* __restrict__ A, int64_t lda, uint16_t* __restrict__ out, int M,
              int K, int kb, int64_t units, int kunits) {
  const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (u >= units) return;
  const int lane = threadIdx.x & 63;
  const int rg = (int)(u / kunits), kg = (int)(u - (int64_t)rg * kunits);
  const int row = rg * 8 + (lane >> 3);
  const int k = kg * 64 + (lane & 7) * 8;
  const int kpad = (K + kb - 1) / kb * kb;
  if (row >= M || k >= kpad) return;
  u32x4 v = {0, 0, 0, 0};
  if (k < K) v = *reinterpret_cast<const u32x4*>(A + (int64_t)row * lda + k);
  *reinterpret_cast<u32x4*>(out + ((int64_t)(k / kb) * M + row) * kb + (k % kb)) = v;
}

// ---------------------------------------------------------------------------
// fp32 kernel: 64x64 tiles, 4 waves of 32x32, v_mfma_f32_16x16x4_f32.
// ---------------------------------------------------------------------------
constexpr int F_BM = 64, F_BN = 64, F_BK = 32;

template <class Epi>
__global__ void __launch_bounds__(256)
gemm_f32_kernel(const float* __restrict__ A, int64_t lda,
                const float* __restrict__ B, int64_t ldb, int M, int N, int K,
                int tiles_m, int tiles_n, Epi epi) {
  __shared__ float As[F_BM][F_BK + 1];
  __shared__ float Bs[F_BK][F_BN + 4];
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * F_BM, n0 = tn * F_BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr0 = (wave >> 1) * 32, wc0 = (wave & 1) * 32;
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0, 0, 0, 0};

  for (int k0 = 0; k0 < K; k0 += F_BK) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int idx = p * 256 + tid;  // 512 float4 in the 64x32 A tile
      const int r = idx >> 3, c = (idx & 7) * 4;
      f32x4 v = f32x4{0, 0, 0, 0};
      if (m0 + r < M && k0 + c < K)
        v = *reinterpret_cast<const f32x4*>(A + (int64_t)(m0 + r) * lda + k0 + c);
      As[r][c] = v[0];
      As[r][c + 1] = v[1];
      As[r][c + 2] = v[2];
      As[r][c + 3] = v[3];
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int idx = p * 256 + tid;  // 512 float4 in the 32x64 B tile
      const int r = idx >> 4, c = (idx & 15) * 4;
      f32x4 v = f32x4{0, 0, 0, 0};
      if (k0 + r < K && n0 + c < N)
        v = *reinterpret_cast<const f32x4*>(B + (int64_t)(k0 + r) * ldb + n0 + c);
      *reinterpret_cast<f32x4*>(&Bs[r][c]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < F_BK; kk += 4) {
      float a[2], b[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) a[mi] = As[wr0 + mi * 16 + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) b[ni] = Bs[kk + (lane >> 4)][wc0 + ni * 16 + (lane & 15)];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
    __syncthreads();
  }
  // 16x16 accumulator layout: lane l, register e holds row 4*(l/16)+e and
  // column l%16 of the block.  Transpose through LDS into runs of 4 columns.
  __shared__ __attribute__((aligned(16))) float stg[4][32][36];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        stg[wave][mi * 16 + 4 * (lane >> 4) + e][ni * 16 + (lane & 15)] = acc[mi][ni][e];
  __syncthreads();
  for (int rr = lane >> 3; rr < 32; rr += 8) {
    const int c4 = (lane & 7) * 4;
    const int row = m0 + wr0 + rr, col0 = n0 + wc0 + c4;
    if (row < M && col0 < N) {
      const f32x4 v4 = *reinterpret_cast<const f32x4*>(&stg[wave][rr][c4]);
      float v[4] = {v4[0], v4[1], v4[2], v4[3]};
      epi.store4(row, col0, v);
    }
  }
}

template <class Epi>
hipError_t launch_f32(const float* A, int64_t lda, const float* B, int64_t ldb,
                      int M, int N, int K, const Epi& epi, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  const int tm = (M + F_BM - 1) / F_BM, tn = (N + F_BN - 1) / F_BN;
  hipLaunchKernelGGL((gemm_f32_kernel<Epi>), dim3(tm * tn), dim3(256), 0, s, A,
                     lda, B, ldb, M, N, K, tm, tn, epi);
  return hipGetLastError();
}

}  // namespace

int device_cu_count() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cached[kMaxDev];  // 0: not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

int gemm_bf16_a_block(int M, int N, int64_t k_split) { return a_block(M, N, k_split); }

int64_t gemm_bf16_split_bytes(int M, int N, int64_t K) { return split_bytes(M, N, K); }

hipError_t gemm_bf16_store_kb(const uint16_t* A, int kb, const uint16_t* B, int64_t ldb,
                              void* C, int64_t ldc, OutType out, int M, int N, int K,
                              float* partials, hipStream_t s) {
  if (M > 0 && N > 0 && kb != a_block(M, N, partials ? K : 0)) return hipErrorInvalidValue;
  return dispatch_bf16<true>(A, M, B, ldb, M, N, K, EpiStore{C, ldc, (int)out}, s, partials);
}

hipError_t kblock_bf16(const uint16_t* A, int64_t lda, uint16_t* out, int M, int K, int kb,
                       hipStream_t s) {
  if ((kb != 32 && kb != 64) || K % 8 || lda % 8) return hipErrorInvalidValue;
  if (M == 0 || K == 0) return hipSuccess;
  const int kpad = (K + kb - 1) / kb * kb;
  const int kunits = (kpad + 63) / 64;
  const int64_t units = (int64_t)((M + 7) / 8) * kunits;
  const int64_t blocks = (units + 3) / 4;
  if (blocks > ((int64_t)1 << 24) - 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kblock_kernel, dim3((unsigned)blocks), dim3(256), 0, s, A, lda, out, M, K,
                     kb, units, kunits);
  return hipGetLastError();
}

hipError_t gemm_bf16_gelu_akb(const uint16_t* Akb, int kb, const uint16_t* B, int64_t ldb,
                              uint16_t* C, int M, int N, int K, int kb_out, hipStream_t s) {
  if (kb_out != 32 && kb_out != 64) return hipErrorInvalidValue;
  if (M > 0 && N > 0 && kb != a_block(M, N, 0)) return hipErrorInvalidValue;
  const int sh = kb_out == 32 ? 5 : 6;
  return dispatch_bf16<true>(Akb, M, B, ldb, M, N, K, EpiGelu{C, 0, M, sh}, s);
}

// The mixed-precision product: 256x256 tiles, K = 32 per stage through a
// 4-slot ring of 32 KB stages (A_hi, B) plus two 16 KB A_lo slots, 160 KB.
hipError_t gemm_f16_bf8_store_kb(const uint8_t* A, const uint16_t* B, int64_t ldb, void* C,
                                 int64_t ldc, OutType out, int M, int N, int K, hipStream_t s) {
  if (K % 64 || ldb >= ((int64_t)1 << 24)) return hipErrorInvalidValue;
  if (M == 0 || N == 0) return hipSuccess;
  const EpiStore epi{C, ldc, (int)out};
  return launch_bf16<256, 256, 2, 2, 2, 4, true, EpiStore, 2>(
      reinterpret_cast<const uint16_t*>(A), M, B, ldb, M, N, K, epi, s);
}

hipError_t gemm_bf16_gelu(const uint16_t* A, int64_t lda, const uint16_t* B,
                          int64_t ldb, uint16_t* C, int64_t ldc, int M, int N,
                          int K, int kb, hipStream_t s) {
  if (kb != 0 && kb != 32 && kb != 64) return hipErrorInvalidValue;
  const int sh = kb == 32 ? 5 : (kb == 64 ? 6 : 0);
  return dispatch_bf16<false>(A, lda, B, ldb, M, N, K, EpiGelu{C, ldc, M, sh}, s);
}

hipError_t gemm_bf16_qkv(const uint16_t* A, int64_t lda, const uint16_t* B,
                         int64_t ldb, const QkvOut& q, int M, int N, int K,
                         hipStream_t s) {
  return dispatch_bf16<false>(A, lda, B, ldb, M, N, K, EpiQkv{q}, s);
}

hipError_t gemm_bf16_add_kb(const uint16_t* A, int kb, const uint16_t* B, int64_t ldb,
                            const float* S, void* C, int64_t ldc, OutType out, int M, int N,
                            int K, float* partials, hipStream_t s) {
  if (M > 0 && N > 0 && kb != a_block(M, N, partials ? K : 0)) return hipErrorInvalidValue;
  return dispatch_bf16<true>(A, M, B, ldb, M, N, K, EpiAdd{S, C, ldc, (int)out}, s, partials);
}

hipError_t gemm_f32_add(const float* A, int64_t lda, const float* B, int64_t ldb,
                        const float* S, void* C, int64_t ldc, OutType out, int M, int N,
                        int K, hipStream_t s) {
  return launch_f32(A, lda, B, ldb, M, N, K, EpiAdd{S, C, ldc, (int)out}, s);
}

hipError_t gemm_f32(const float* A, int64_t lda, const float* B, int64_t ldb,
                    void* C, int64_t ldc, OutType out, bool gelu, int M, int N,
                    int K, hipStream_t s) {
  if (gelu) {
    if (out != OUT_F32) return hipErrorInvalidValue;  // GeLU(Z) stays fp32 on this path
    return launch_f32(A, lda, B, ldb, M, N, K, EpiGeluF32{static_cast<float*>(C), ldc}, s);
  }
  return launch_f32(A, lda, B, ldb, M, N, K, EpiStore{C, ldc, (int)out}, s);
}

}  // namespace tp
