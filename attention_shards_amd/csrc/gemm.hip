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
//   * gemm_bf16_kernel: 4 waves, 256x128, 128x192 or 128x128 tiles, K = 64
//     per stage through a 3-slot ring, DMAs and fragment reads interleaved
//     between the MFMAs of each wave.  (128x192 fills all 256 CUs where
//     256x128 would leave a quarter idle, e.g. 2048 x 3072 outputs.)
//   * gemm_bf16_pp_kernel: 8 waves, 256x256 tiles, K = 32 per stage through
//     a 5-slot ring; two groups of waves alternate between a memory phase and
//     an MFMA-only phase, one phase apart, so each SIMD's matrix pipe is fed
//     by one wave or the other.
//   * Workgroup ids are remapped so each XCD (dispatch is round-robin over
//     the 8 XCDs) receives a contiguous run of tiles, ordered in groups of 8
//     tile-rows so neighbouring tiles share A and B panels in that XCD's L2.
#include "internal.h"

namespace tp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Two fp32 values rounded to bf16 (nearest even) and packed, low half
// first: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// GeLU(z) = z * Phi(z), Phi the standard normal CDF, with Phi from erfc
// through the rational approximation of Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (|error of erf| <= 1.5e-7 for
// x >= 0): erfc(x) = t P(t) exp(-x^2), t = 1/(1 + 0.3275911 x), taken at
// x = |z|/sqrt(2).  With E = z erfc(x)/2 (the sign of z), GeLU = z - E for
// z >= 0 and E for z < 0, i.e. max(z, 0) - |E|.  Branch-free: one
// reciprocal, one exponential, ten multiply(-add)s, a max and a subtract;
// P/2's coefficients are P's halved (exact), so |GeLU error| <= |z| * 1e-7
// plus fp32 rounding.
__device__ __forceinline__ float gelu_erf(float z) {
  const float t = __builtin_amdgcn_rcpf(fmaf(fabsf(z), 0.3275911f * 0.70710678118654752f, 1.0f));
  float p = fmaf(0.5307027145f, t, -0.7265760135f);
  p = fmaf(p, t, 0.7107068705f);
  p = fmaf(p, t, -0.142248368f);
  p = fmaf(p, t, 0.127414796f);
  const float e = __builtin_amdgcn_exp2f(z * z * (-0.5f * 1.4426950408889634f));
  const float E = z * (p * t * e);
  return fmaxf(z, 0.0f) - fabsf(E);
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

// GeLU(acc), row-major (row stride ldc) or, with kb_shift > 0 and bf16
// output, K-blocked for the next product: column c of row r at
// ((c >> kb_shift) * rows + r) * kb + c % kb, kb = 1 << kb_shift, so that
// each kb-column block of all rows is one contiguous [rows][kb] slab.
struct EpiGelu {
  void* C;
  int64_t ldc;
  int out;
  int rows;
  int kb_shift;
  __device__ int64_t kblock_at(int row, int col0) const {
    const int kb = 1 << kb_shift;
    return ((int64_t)(col0 >> kb_shift) * rows + row) * kb + (col0 & (kb - 1));
  }
  __device__ void store4(int row, int col0, const float* v) const {
    float g[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) g[r] = gelu_erf(v[r]);
    if (kb_shift)
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(C) + kblock_at(row, col0)) =
          uint2{pack_bf16(g[0], g[1]), pack_bf16(g[2], g[3])};
    else
      store_run4(C, ldc, out, row, col0, g);
  }
  __device__ void store8(int row, int col0, const float* v) const {
    float g[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) g[r] = gelu_erf(v[r]);
    if (kb_shift)
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(C) + kblock_at(row, col0)) =
          u32x4{pack_bf16(g[0], g[1]), pack_bf16(g[2], g[3]), pack_bf16(g[4], g[5]),
                pack_bf16(g[6], g[7])};
    else
      store_run8(C, ldc, out, row, col0, g);
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

// Rows per epilogue call in the GEMM's store loop (see the kernel).
template <class E>
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
      // bf16 hi/lo pair: hi = bf16(v), lo = bf16(v - hi)
      const uint32_t h01 = pack_bf16(v[0], v[1]), h23 = pack_bf16(v[2], v[3]);
      const uint32_t l01 = pack_bf16(v[0] - __uint_as_float(h01 << 16),
                                     v[1] - __uint_as_float(h01 & 0xFFFF0000u));
      const uint32_t l23 = pack_bf16(v[2] - __uint_as_float(h23 << 16),
                                     v[3] - __uint_as_float(h23 & 0xFFFF0000u));
      const int64_t off = (bh * q.seq_pad + s) * 128 + dd;
      uint16_t* ph = sec == 0 ? q.q_hi : q.k_hi;
      uint16_t* pl = sec == 0 ? q.q_lo : q.k_lo;
      *reinterpret_cast<uint2*>(ph + off) = uint2{h01, h23};
      *reinterpret_cast<uint2*>(pl + off) = uint2{l01, l23};
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
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm,
                                            int& tn) {
  const int bid = blockIdx.x;
  const int nb = gridDim.x;
  const int xcd = bid & 7, j = bid >> 3, q = nb >> 3, r = nb & 7;
  const int lin = xcd * q + (xcd < r ? xcd : r) + j;
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int g = lin / per_group;
  const int first_m = g * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int w = lin - g * per_group;
  tm = first_m + w % gsize;
  tn = w / gsize;
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
// fewer, larger ring slots.
template <int BM, int BN, int WM, int WN, int KS, int NSL, class Epi, bool AKB>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_bf16_kernel(const uint16_t* __restrict__ A, int64_t lda,
                 const uint16_t* __restrict__ B, int64_t ldb, int M, int N,
                 int K, int kwrap, int tiles_m, int tiles_n, Epi epi) {
  // Stage kt reads B rows from (k0 < kwrap ? k0 : k0 - kwrap); with kwrap < K
  // (K == 2 kwrap, kwrap a multiple of BK) the same B multiplies both halves
  // of an A laid out as [A_hi | A_lo].  With AKB, A is K-blocked by the
  // stage depth BK: [ceil(K/BK)][lda][BK], lda the padded row count, so a
  // stage's A tile is one contiguous run of rows.
  static_assert(KS == 2 || KS == 4, "k-steps per stage");
  static_assert(NSL >= 3 && NSL <= 6, "ring slots");
  constexpr int BK = 16 * KS;
  constexpr int NW = WM * WN;
  constexpr int FM = BM / WM / 32;
  constexpr int FN = BN / WN / 32;
  constexpr int A_ROWB = BK * 2;           // A rows in LDS: 64 or 128 bytes
  constexpr int CPR = A_ROWB / 16;         // 16-byte chunks per A row (4 or 8)
  constexpr int RPD = 64 / CPR;            // A rows per 1 KiB DMA
  constexpr int ASH = CPR == 4 ? 2 : 1;    // A swizzle: chunk ^ ((row >> ASH) & (CPR-1))
  constexpr int B_ROWB = BN * 2;           // B rows in LDS: natural [k][n]
  constexpr int B_CH = B_ROWB / 16;        // 16-byte chunks per B row
  constexpr int A_STAGE = BM * A_ROWB;
  constexpr int B_STAGE = BK * B_ROWB;
  constexpr int A_DMA = A_STAGE / 1024 / NW;  // 1 KiB DMAs per wave per stage
  constexpr int B_DMA = B_STAGE / 1024 / NW;
  constexpr int NDMA = A_DMA + B_DMA;
  static_assert(A_DMA * 1024 * NW == A_STAGE && B_DMA * 1024 * NW == B_STAGE, "DMA split");
  static_assert(B_CH % 16 == 0 || B_CH == 24, "B swizzle: 256-byte multiple or 384-byte rows");
  static_assert(FM >= 1 && FN >= 1, "wave tile");

  // LDS ring: slot s holds A at s*A_STAGE and B at NSL*A_STAGE + s*B_STAGE.
  // The same memory later stages the epilogue (NW regions of 32 x (BN/WN+4)).
  constexpr int PIPE_BYTES = NSL * (A_STAGE + B_STAGE);
  constexpr int EPI_BYTES = NW * 32 * (BN / WN + 4) * 4;
  __shared__ __attribute__((aligned(16))) uint8_t
      smem[PIPE_BYTES > EPI_BYTES ? PIPE_BYTES : EPI_BYTES];
  uint8_t* const lds_a = smem;
  uint8_t* const lds_b = smem + NSL * A_STAGE;
  const uint32_t lds_a_addr = (uint32_t)(uintptr_t)(lds_u8*)lds_a;
  const uint32_t lds_b_addr = (uint32_t)(uintptr_t)(lds_u8*)lds_b;

  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
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

  // DMA number j (0 <= j < NDMA) of stage kt into ring slot SLOT.
  auto dma = [&](int kt, auto SLOT, int j) {
    constexpr int slot = decltype(SLOT)::value;
    const int k0 = kt * BK;
    if (j < A_DMA) {
      const __amdgpu_buffer_rsrc_t ra =
          AKB ? make_rsrc(A + ((int64_t)kt * lda + m0) * BK, (int64_t)rows_valid * A_ROWB)
              : make_rsrc(A + (int64_t)m0 * lda + k0, (int64_t)rows_valid * lda * 2 - (int64_t)k0 * 2);
      const int off = (k0 + a_col[j] < K) ? a_off[j] : OOB;
      dma16(ra, off, lds_a_addr + slot * A_STAGE + (j * NW + wave) * 1024);
    } else {
      const int jb = j - A_DMA;
      const int bk0 = k0 < kwrap ? k0 : k0 - kwrap;
      const int rows_left = (k0 < kwrap ? kwrap : K) - k0;
      const __amdgpu_buffer_rsrc_t rb =
          make_rsrc(B + (int64_t)bk0 * ldb + n0,
                    ((int64_t)rows_left - 1) * ldb * 2 + (int64_t)cols_valid * 2);
      dma16(rb, b_off[jb], lds_b_addr + slot * B_STAGE + (jb * NW + wave) * 1024);
    }
  };

  // ---- fragment read addresses (byte offsets inside a slot).
  // A (ds_read_b128): row wr0 + mi*32 + (lane&31), chunk 2ks + (lane>>5).
  int a_rd[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c = (2 * ks + (lane >> 5)) ^ (((lane & 31) >> ASH) & (CPR - 1));
    a_rd[ks] = (wr0 + (lane & 31)) * A_ROWB + c * 16;
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

  bf16x8 fa[2][FM], fb[2][FN];
  // Fragment read unit q of k-step ks from ring slot SLOT into set fset:
  // units 0..FN-1 are B fragments (two transposed reads each), units
  // FN..FN+FM-1 are A fragments.
  auto read_unit = [&](auto SLOT, int ks, int fset, int q) {
    constexpr int slot = decltype(SLOT)::value;
    if (q < FN) {
      const uint8_t* lb = lds_b + slot * B_STAGE + ks * 16 * B_ROWB + b_rd[q];
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)lb);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(lb + 4 * B_ROWB));
      fb[fset][q] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      const int mi = q - FN;
      fa[fset][mi] = *reinterpret_cast<const bf16x8*>(lds_a + slot * A_STAGE + a_rd[ks] +
                                                     mi * 32 * A_ROWB);
    }
  };
  auto mfma1 = [&](int fset, int idx) {  // one MFMA of a k-step, idx in [0, FM*FN)
    const int mi = idx / FN, ni = idx % FN;
    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[fset][mi], fb[fset][ni],
                                                          acc[mi][ni], 0, 0, 0);
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
  constexpr int NMF = FM * FN;   // MFMAs per k-step
  constexpr int NRU = FM + FN;   // fragment read units per k-step
  constexpr int DSLOTS = (KS - 1) * NMF;
  static_assert(NDMA <= DSLOTS && NRU <= NMF, "traffic fits between the MFMAs");
  // MFMA slot after which DMA d of a step is issued
  auto dma_slot = [](int d) { return KS == 2 ? NMF - NDMA + d : d * DSLOTS / NDMA; };
  auto step = [&](int kt, auto U) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    constexpr int nxt = (u + NSL - 1) % NSL;
#pragma unroll
    for (int ksi = 0; ksi < KS - 1; ++ksi) {
#pragma unroll
      for (int j = 0; j < NMF; ++j) {
        mfma1(ksi & 1, j);
        __builtin_amdgcn_sched_barrier(0);
        if (j < NRU) read_unit(IC<u>{}, ksi + 1, (ksi + 1) & 1, j);
#pragma unroll
        for (int d = 0; d < NDMA; ++d)
          if (dma_slot(d) == ksi * NMF + j) dma(kt + NSL - 1, IC<nxt>{}, d);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_vmcnt<(NSL - 2) * NDMA>();
    wait_lgkmcnt0();
    stage_barrier();
#pragma unroll
    for (int j = 0; j < NMF; ++j) {
      mfma1((KS - 1) & 1, j);
      __builtin_amdgcn_sched_barrier(0);
      if (j < NRU) read_unit(IC<(u + 1) % NSL>{}, 0, 0, j);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue: stages 0..NSL-2 in flight, wait for stage 0.
  static_for<0, NSL - 1>([&](auto S) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NDMA; ++j) dma(decltype(S)::value, S, j);
  });
  wait_vmcnt<(NSL - 2) * NDMA>();
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

  epilogue_lds<BN / WN>(smem, acc, epi, M, N, m0 + wr0, n0 + wc0, wave, lane);
}

// 256x256 tiles with eight waves in two groups that take turns on the
// matrix cores ("ping-pong").  Waves w and w+4 share SIMD w%4; group 0
// (waves 0-3) owns output rows 0-127 and group 1 rows 128-255, each wave a
// 128x64 block (4x2 accumulator blocks of v_mfma_f32_32x32x16_bf16).  K
// advances in stages of 32 through a five-slot LDS ring (32 KB per stage,
// the same layout and swizzles as gemm_bf16_kernel with KS = 2).  Every wave
// alternates two phases separated by workgroup barriers:
//   mem(s):  issue its share of the DMAs of stage s+4 (into the slot that
//            stage s-1 freed), read all of its fragments of stage s, then
//            wait until its own DMAs of stage s+1 and its LDS reads are done;
//   comp(s): 16 MFMAs on those fragments and nothing else.
// Group 1 starts one phase late, so while one wave of a SIMD runs its MFMAs
// the other loads; the matrix pipe is fed by one wave or the other in every
// phase.  With phases numbered from 0, group 0 runs mem(s) in phase 2s and
// comp(s) in 2s+1, group 1 one phase later.  Ring safety: slot s%5 is read in
// phases 2s (group 0) and 2s+1 (group 1), each wave waiting for its reads
// before the barrier that ends its mem phase, and is refilled (stage s+5)
// from phase 2s+2 on; stage s+1 is read from phase 2s+2 on and every wave has
// waited for its share of it by the end of phase 2s+1.
template <class Epi, bool AKB>
__global__ void __launch_bounds__(512)
gemm_bf16_pp_kernel(const uint16_t* __restrict__ A, int64_t lda,
                    const uint16_t* __restrict__ B, int64_t ldb, int M, int N,
                    int K, int kwrap, int tiles_m, int tiles_n, Epi epi) {
  constexpr int BM = 256, BN = 256, NW = 8, WN = 4;
  constexpr int BK = 32, NSL = 5;
  constexpr int FM = 4, FN = 2;            // 128 x 64 per wave
  constexpr int A_ROWB = BK * 2;           // 64-byte A rows
  constexpr int CPR = 4, RPD = 16, ASH = 2;
  constexpr int B_ROWB = BN * 2;           // 512-byte B rows
  constexpr int B_CH = B_ROWB / 16;
  constexpr int A_STAGE = BM * A_ROWB;     // 16 KB
  constexpr int B_STAGE = BK * B_ROWB;     // 16 KB
  constexpr int A_DMA = A_STAGE / 1024 / NW;  // 2
  constexpr int B_DMA = B_STAGE / 1024 / NW;  // 2
  constexpr int NDMA = A_DMA + B_DMA;
  static_assert(A_DMA * 1024 * NW == A_STAGE && B_DMA * 1024 * NW == B_STAGE, "DMA split");

  __shared__ __attribute__((aligned(16))) uint8_t smem[NSL * (A_STAGE + B_STAGE)];
  static_assert(NW * 32 * (BN / WN + 4) * 4 <= (int)sizeof(smem), "epilogue staging fits");
  uint8_t* const lds_a = smem;
  uint8_t* const lds_b = smem + NSL * A_STAGE;
  const uint32_t lds_a_addr = (uint32_t)(uintptr_t)(lds_u8*)lds_a;
  const uint32_t lds_b_addr = (uint32_t)(uintptr_t)(lds_u8*)lds_b;

  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wr0 = grp * 128;
  const int wc0 = (wave & 3) * 64;
  const int rows_valid = min(BM, M - m0);
  const int cols_valid = min(BN, N - n0);

  // DMA lane offsets (as in gemm_bf16_kernel).
  int a_off[A_DMA], a_col[A_DMA];
#pragma unroll
  for (int j = 0; j < A_DMA; ++j) {
    const int row = RPD * (j * NW + wave) + lane / CPR;
    const int c = (lane % CPR) ^ ((row >> ASH) & (CPR - 1));
    a_off[j] = AKB ? row * A_ROWB + c * 16 : row * (int)lda * 2 + c * 16;
    a_col[j] = c * 8;
  }
  int b_off[B_DMA];
#pragma unroll
  for (int j = 0; j < B_DMA; ++j) {
    const int row = (j * NW + wave) * (1024 / B_ROWB) + lane / B_CH;
    const int c = (lane % B_CH) ^ ((row & 3) << 2);
    b_off[j] = row * (int)ldb * 2 + c * 16;
  }
  // All of this wave's DMAs of stage kt into ring slot `slot`.
  auto dma_stage = [&](int kt, int slot) __attribute__((always_inline)) {
    const int k0 = kt * BK;
    const __amdgpu_buffer_rsrc_t ra =
        AKB ? make_rsrc(A + ((int64_t)kt * lda + m0) * BK, (int64_t)rows_valid * A_ROWB)
            : make_rsrc(A + (int64_t)m0 * lda + k0, (int64_t)rows_valid * lda * 2 - (int64_t)k0 * 2);
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) {
      const int off = (k0 + a_col[j] < K) ? a_off[j] : OOB;
      dma16(ra, off, lds_a_addr + slot * A_STAGE + (j * NW + wave) * 1024);
    }
    const int bk0 = k0 < kwrap ? k0 : k0 - kwrap;
    const int rows_left = (k0 < kwrap ? kwrap : K) - k0;
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(B + (int64_t)bk0 * ldb + n0,
                  ((int64_t)rows_left - 1) * ldb * 2 + (int64_t)cols_valid * 2);
#pragma unroll
    for (int j = 0; j < B_DMA; ++j)
      dma16(rb, b_off[j], lds_b_addr + slot * B_STAGE + (j * NW + wave) * 1024);
  };

  // Fragment read offsets inside a slot (as in gemm_bf16_kernel).
  int a_rd[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int c = (2 * ks + (lane >> 5)) ^ (((lane & 31) >> ASH) & (CPR - 1));
    a_rd[ks] = (wr0 + (lane & 31)) * A_ROWB + c * 16;
  }
  int b_rd[FN];
  {
    const int G = lane >> 4, r = lane & 15;
    const int krow = 8 * (G >> 1) + (r >> 2);
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
      const int c = (((wc0 + ni * 32) >> 3) + 2 * (G & 1) + ((r & 3) >> 1)) ^ ((r >> 2) << 2);
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

  bf16x8 fa[2][FM], fb[2][FN];
  auto read_stage = [&](int slot) __attribute__((always_inline)) {
    const uint8_t* la = lds_a + slot * A_STAGE;
    const uint8_t* lb = lds_b + slot * B_STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
        fa[ks][mi] = *reinterpret_cast<const bf16x8*>(la + a_rd[ks] + mi * 32 * A_ROWB);
#pragma unroll
      for (int ni = 0; ni < FN; ++ni) {
        const uint8_t* p = lb + ks * 16 * B_ROWB + b_rd[ni];
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)p);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(p + 4 * B_ROWB));
        fb[ks][ni] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };

  const int nk = (K + BK - 1) / BK;

  // Prologue: stages 0..NSL-2 in flight, wait for stage 0.
#pragma unroll
  for (int q = 0; q < NSL - 1; ++q) dma_stage(q, q);
  wait_vmcnt<(NSL - 2) * NDMA>();
  stage_barrier();
  if (grp == 1) stage_barrier();
  int slot = 0;                 // s % NSL
  int fill = NSL - 1;           // (s + NSL - 1) % NSL
  for (int s = 0; s < nk; ++s) {
    // mem(s)
    dma_stage(s + NSL - 1, fill);
    read_stage(slot);
    wait_vmcnt<(NSL - 2) * NDMA>();
    wait_lgkmcnt0();
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // comp(s)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks][mi], fb[ks][ni],
                                                                acc[mi][ni], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    stage_barrier();
    slot = slot == NSL - 1 ? 0 : slot + 1;
    fill = fill == NSL - 1 ? 0 : fill + 1;
  }
  if (grp == 0) stage_barrier();
  wait_vmcnt<0>();
  __syncthreads();

  epilogue_lds<BN / WN>(smem, acc, epi, M, N, m0 + wr0, n0 + wc0, wave, lane);
}

// Tile configurations.  The choice minimises the estimated time: full
// 256-CU waves of tiles times the tile's cost, the larger tiles being
// cheaper per element (less LDS and L2 traffic per MFMA).
struct TileChoice {
  int bm, bn;
};

TileChoice choose_bf16_tile(int M, int N) {
  const TileChoice cand[4] = {{256, 256}, {256, 128}, {128, 192}, {128, 128}};
  const double eff[4] = {1.0, 0.95, 0.80, 0.70};
  int best = 0;
  double best_cost = 1e300;
  for (int c = 0; c < 4; ++c) {
    const int64_t tiles = (int64_t)((M + cand[c].bm - 1) / cand[c].bm) *
                          ((N + cand[c].bn - 1) / cand[c].bn);
    const double waves = (double)((tiles + 255) / 256);
    const double cost = waves * cand[c].bm * cand[c].bn / eff[c];
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = c;
    }
  }
  return cand[best];
}

template <int BM, int BN, int WM, int WN, int KS, int NSL, bool AKB, class Epi>
hipError_t launch_bf16(const uint16_t* A, int64_t lda, const uint16_t* B,
                       int64_t ldb, int M, int N, int K, int kwrap,
                       const Epi& epi, hipStream_t s) {
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, KS, NSL, Epi, AKB>), dim3(tm * tn),
                     dim3(WM * WN * 64), 0, s, A, lda, B, ldb, M, N, K, kwrap,
                     tm, tn, epi);
  return hipGetLastError();
}

// K block (stage depth) of the kernel the dispatch picks for an [M, N]
// output: 32 for the 256x256 ping-pong kernel, 64 for the others.
int a_block(const TileChoice& t) { return t.bm == 256 && t.bn == 256 ? 32 : 64; }

// AKB: A is K-blocked by the chosen kernel's stage depth (see
// gemm_bf16_kernel), lda its row count; the caller has checked the block.
template <bool AKB, class Epi>
hipError_t dispatch_bf16(const uint16_t* A, int64_t lda, const uint16_t* B,
                         int64_t ldb, int M, int N, int K, int kwrap,
                         const Epi& epi, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  // tiles are addressed with 32-bit byte offsets: 256 rows of A, 64 of B
  // (K-blocked A tiles are at most 32 KiB)
  if ((!AKB && lda >= ((int64_t)1 << 22)) || ldb >= ((int64_t)1 << 24)) return hipErrorInvalidValue;
  const TileChoice t = choose_bf16_tile(M, N);
  if (t.bm == 256 && t.bn == 256) {
    const int tm = (M + 255) / 256, tn = (N + 255) / 256;
    hipLaunchKernelGGL((gemm_bf16_pp_kernel<Epi, AKB>), dim3(tm * tn), dim3(512), 0, s, A, lda,
                       B, ldb, M, N, K, kwrap, tm, tn, epi);
    return hipGetLastError();
  }
  if (t.bm == 256 && t.bn == 128)
    return launch_bf16<256, 128, 2, 2, 4, 3, AKB>(A, lda, B, ldb, M, N, K, kwrap, epi, s);
  if (t.bm == 128 && t.bn == 192)
    return launch_bf16<128, 192, 2, 2, 4, 3, AKB>(A, lda, B, ldb, M, N, K, kwrap, epi, s);
  return launch_bf16<128, 128, 2, 2, 4, 3, AKB>(A, lda, B, ldb, M, N, K, kwrap, epi, s);
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

int gemm_bf16_a_block(int M, int N) { return a_block(choose_bf16_tile(M, N)); }

hipError_t gemm_bf16_store_kb(const uint16_t* A, int kb, const uint16_t* B, int64_t ldb,
                              void* C, int64_t ldc, OutType out, int M, int N, int K,
                              hipStream_t s) {
  if (M > 0 && N > 0 && kb != a_block(choose_bf16_tile(M, N))) return hipErrorInvalidValue;
  return dispatch_bf16<true>(A, M, B, ldb, M, N, K, K, EpiStore{C, ldc, (int)out}, s);
}

hipError_t gemm_bf16_store_split_a_kb(const uint16_t* A2, int kb, const uint16_t* B,
                                      int64_t ldb, void* C, int64_t ldc, OutType out, int M,
                                      int N, int K, hipStream_t s) {
  if (K % 64) return hipErrorInvalidValue;
  if (M > 0 && N > 0 && kb != a_block(choose_bf16_tile(M, N))) return hipErrorInvalidValue;
  return dispatch_bf16<true>(A2, M, B, ldb, M, N, 2 * K, K, EpiStore{C, ldc, (int)out}, s);
}

hipError_t gemm_bf16_gelu(const uint16_t* A, int64_t lda, const uint16_t* B,
                          int64_t ldb, uint16_t* C, int64_t ldc, int M, int N,
                          int K, int kb, hipStream_t s) {
  if (kb != 0 && kb != 32 && kb != 64) return hipErrorInvalidValue;
  const int sh = kb == 32 ? 5 : (kb == 64 ? 6 : 0);
  return dispatch_bf16<false>(A, lda, B, ldb, M, N, K, K, EpiGelu{C, ldc, (int)OUT_BF16, M, sh}, s);
}

hipError_t gemm_bf16_qkv(const uint16_t* A, int64_t lda, const uint16_t* B,
                         int64_t ldb, const QkvOut& q, int M, int N, int K,
                         hipStream_t s) {
  return dispatch_bf16<false>(A, lda, B, ldb, M, N, K, K, EpiQkv{q}, s);
}

hipError_t gemm_bf16_add_kb(const uint16_t* A, int kb, const uint16_t* B, int64_t ldb,
                            const float* S, void* C, int64_t ldc, OutType out, int M, int N,
                            int K, hipStream_t s) {
  if (M > 0 && N > 0 && kb != a_block(choose_bf16_tile(M, N))) return hipErrorInvalidValue;
  return dispatch_bf16<true>(A, M, B, ldb, M, N, K, K, EpiAdd{S, C, ldc, (int)out}, s);
}

hipError_t gemm_f32_add(const float* A, int64_t lda, const float* B, int64_t ldb,
                        const float* S, void* C, int64_t ldc, OutType out, int M, int N,
                        int K, hipStream_t s) {
  return launch_f32(A, lda, B, ldb, M, N, K, EpiAdd{S, C, ldc, (int)out}, s);
}

hipError_t gemm_f32(const float* A, int64_t lda, const float* B, int64_t ldb,
                    void* C, int64_t ldc, OutType out, bool gelu, int M, int N,
                    int K, hipStream_t s) {
  if (gelu) return launch_f32(A, lda, B, ldb, M, N, K, EpiGelu{C, ldc, (int)out, 0, 0}, s);
  return launch_f32(A, lda, B, ldb, M, N, K, EpiStore{C, ldc, (int)out}, s);
}

}  // namespace tp
