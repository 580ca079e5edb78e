// Sum of the t shard partials plus the residual, in HBM on one GPU:
//     out = ((P_0 + P_1) + ... + P_{t-1}) + R
// This is the arithmetic of the all-reduce of FFN step 3 followed by the
// residual add of the closing paragraph (page "Tensor Parallelism >
// Combining Column and Row Parallelism"), without any transfer between GPUs.
//
// Pure streaming, HBM-bound: each thread owns runs of 8 elements (16-byte
// bf16 vectors, 2 x 16-byte fp32 vectors), loads the same run of up to
// eight partials and the residual before adding (all loads in flight),
// accumulates in fp32 in the fixed order above and rounds once.  Inputs are read with non-temporal
// loads and the output is written with non-temporal stores, so a reduce of
// buffers larger than the caches does not evict anything useful.
#include "internal.h"

namespace tp {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum { DT_F32 = 0, DT_BF16 = 1, DT_NONE = 2 };

__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t g, float* v) {
  if (DT == DT_BF16) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + g);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(base) + 2 * g;
    const f32x4 a = __builtin_nontemporal_load(p);
    const f32x4 b = __builtin_nontemporal_load(p + 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = a[k];
      v[4 + k] = b[k];
    }
  }
}

// The same 8 elements as load8, split into the load (raw bits, so several
// can be issued before any is needed) and the conversion.
struct Raw8 {
  f32x4 a, b;  // fp32: elements 0-3, 4-7; bf16: a holds the 8 values' bits
};

template <int DT>
__device__ __forceinline__ Raw8 rawload8(const void* base, int64_t g) {
  Raw8 r;
  if (DT == DT_BF16) {
    r.a = __builtin_bit_cast(f32x4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + g));
    r.b = f32x4{0, 0, 0, 0};
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(base) + 2 * g;
    r.a = __builtin_nontemporal_load(p);
    r.b = __builtin_nontemporal_load(p + 1);
  }
  return r;
}

template <int DT>
__device__ __forceinline__ void unpack8(const Raw8& r, float* v) {
  if (DT == DT_BF16) {
    const u32x4 w = __builtin_bit_cast(u32x4, r.a);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = r.a[k];
      v[4 + k] = r.b[k];
    }
  }
}

template <int DT>
__device__ __forceinline__ void add8(const Raw8& r, float* acc) {
  float v[8];
  unpack8<DT>(r, v);
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] += v[k];
}

template <int DT>
__device__ __forceinline__ void store8(void* base, int64_t g, const float* v) {
  if (DT == DT_BF16) {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = f2bf(v[2 * k]) | (f2bf(v[2 * k + 1]) << 16);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(base) + g);
  } else {
    f32x4* p = reinterpret_cast<f32x4*>(base) + 2 * g;
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, p);
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, p + 1);
  }
}

template <int DT>
__device__ __forceinline__ float load1(const void* base, int64_t k) {
  if (DT == DT_BF16)
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[k] << 16);
  return static_cast<const float*>(base)[k];
}

template <int DT>
__device__ __forceinline__ void store1(void* base, int64_t k, float v) {
  if (DT == DT_BF16)
    static_cast<uint16_t*>(base)[k] = (uint16_t)f2bf(v);
  else
    static_cast<float*>(base)[k] = v;
}

template <int PDT, int RDT, int ODT, int C>
__global__ void __launch_bounds__(256)
reduce_kernel(ReducePtrs ptrs, int t, const void* R,
              void* out, int64_t ngroups, int tail) {
  // the last `tail` (< 8) elements, one per thread of block 0, same order
  if (blockIdx.x == 0 && (int)threadIdx.x < tail) {
    const int64_t k = ngroups * 8 + threadIdx.x;
    float acc = load1<PDT>(ptrs.p[0], k);
    for (int i = 1; i < t; ++i) acc += load1<PDT>(ptrs.p[i], k);
    if (RDT != DT_NONE) acc += load1<RDT>(R, k);
    store1<ODT>(out, k, acc);
  }
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x; gi < ngroups; gi += stride) {
    // Partial 0 and partials 1..C, then further chunks of C: all loads of
    // a chunk (with the last chunk, the residual's too) are issued before
    // the first add.  A chunk that runs past t re-reads partial t-1 (a
    // cache hit) and skips the add, so no load sits under a branch.  The
    // adds follow the fixed order.
    float acc[8];
    {
      const bool last = 1 + C >= t;
      Raw8 rr;
      if (RDT != DT_NONE) rr = rawload8<RDT>(R, last ? gi : 0);
      const Raw8 r0 = rawload8<PDT>(ptrs.p[0], gi);
      Raw8 v[C];
#pragma unroll
      for (int u = 0; u < C; ++u) v[u] = rawload8<PDT>(ptrs.p[1 + u < t ? 1 + u : t - 1], gi);
      unpack8<PDT>(r0, acc);
#pragma unroll
      for (int u = 0; u < C; ++u)
        if (1 + u < t) add8<PDT>(v[u], acc);
      if (RDT != DT_NONE && last) add8<RDT>(rr, acc);
    }
    for (int i0 = 1 + C; i0 < t; i0 += C) {
      const bool last = i0 + C >= t;
      Raw8 rr;
      if (RDT != DT_NONE) rr = rawload8<RDT>(R, last ? gi : 0);
      Raw8 v[C];
#pragma unroll
      for (int u = 0; u < C; ++u) v[u] = rawload8<PDT>(ptrs.p[i0 + u < t ? i0 + u : t - 1], gi);
#pragma unroll
      for (int u = 0; u < C; ++u)
        if (i0 + u < t) add8<PDT>(v[u], acc);
      if (RDT != DT_NONE && last) add8<RDT>(rr, acc);
    }
    store8<ODT>(out, gi, acc);
  }
}

template <int PDT, int RDT, int ODT, int C>
hipError_t launch_c(const ReducePtrs& ptrs, int t, const void* R, void* out,
                    int64_t n, hipStream_t s) {
  const int64_t ngroups = n / 8;
  // One 8-element group per thread (measured on MI355X with inputs rotated
  // through more memory than the caches hold: t=8 bf16 [4096,4096] 5.9 TB/s
  // vs 5.7 TB/s for a grid capped at 4096 looping blocks).
  // The grid-stride loop covers what a grid of at most 2^24 - 1 blocks
  // (below the 2^32 work-items a dispatch may hold) does not.
  int64_t blocks = (ngroups + 255) / 256;
  if (blocks > ((int64_t)1 << 24) - 1) blocks = ((int64_t)1 << 24) - 1;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((reduce_kernel<PDT, RDT, ODT, C>), dim3((unsigned)blocks),
                     dim3(256), 0, s, ptrs, t, R, out, ngroups, (int)(n - ngroups * 8));
  return hipGetLastError();
}

// Chunk size: t-1 for t <= 8, so the first chunk holds exactly the later
// partials and no load is a duplicate (fp32 partials at t=8 [2048,8192]:
// 5.7 vs 5.3 TB/s with one duplicate per group); chunks of 8 beyond.
template <int PDT, int RDT, int ODT>
hipError_t launch(const ReducePtrs& ptrs, int t, const void* R, void* out,
                  int64_t n, hipStream_t s) {
  switch (t) {
    case 1:
    case 2: return launch_c<PDT, RDT, ODT, 1>(ptrs, t, R, out, n, s);
    case 3: return launch_c<PDT, RDT, ODT, 2>(ptrs, t, R, out, n, s);
    case 4: return launch_c<PDT, RDT, ODT, 3>(ptrs, t, R, out, n, s);
    case 5: return launch_c<PDT, RDT, ODT, 4>(ptrs, t, R, out, n, s);
    case 6: return launch_c<PDT, RDT, ODT, 5>(ptrs, t, R, out, n, s);
    case 7: return launch_c<PDT, RDT, ODT, 6>(ptrs, t, R, out, n, s);
    case 8: return launch_c<PDT, RDT, ODT, 7>(ptrs, t, R, out, n, s);
    default: return launch_c<PDT, RDT, ODT, 8>(ptrs, t, R, out, n, s);
  }
}

template <int PDT, int RDT>
hipError_t launch_o(const ReducePtrs& ptrs, int t, const void* R, void* out,
                    int odt, int64_t n, hipStream_t s) {
  return odt == DT_BF16 ? launch<PDT, RDT, DT_BF16>(ptrs, t, R, out, n, s)
                        : launch<PDT, RDT, DT_F32>(ptrs, t, R, out, n, s);
}

template <int PDT>
hipError_t launch_r(const ReducePtrs& ptrs, int t, const void* R, int rdt,
                    void* out, int odt, int64_t n, hipStream_t s) {
  if (R == nullptr) return launch_o<PDT, DT_NONE>(ptrs, t, R, out, odt, n, s);
  return rdt == DT_BF16 ? launch_o<PDT, DT_BF16>(ptrs, t, R, out, odt, n, s)
                        : launch_o<PDT, DT_F32>(ptrs, t, R, out, odt, n, s);
}

}  // namespace

hipError_t partial_reduce(const ReducePtrs& ptrs, int t, int pdt, const void* R,
                          int rdt, void* out, int odt, int64_t n,
                          hipStream_t s) {
  if (n == 0) return hipSuccess;
  return pdt == DT_BF16 ? launch_r<DT_BF16>(ptrs, t, R, rdt, out, odt, n, s)
                        : launch_r<DT_F32>(ptrs, t, R, rdt, out, odt, n, s);
}


// ---------------------------------------------------------------------------
// Sequence-parallel sum + LayerNorm: a block of rows of out = sum_i P_i + R
// (the reduce-scatter half of the all-reduce, split by rows), then LayerNorm
// over each of those full-width rows (page "Tensor Parallelism > Combining
// Column and Row Parallelism": LayerNorm reduces over all features, so it is
// not split by columns; the rows are split instead).
//
// One workgroup per row, nt threads (a multiple of 64, at most 1024); thread
// k owns the 8-element groups k, k + nt, ... (G of them) and loads each the
// way reduce_kernel loads its group: partial 0 and the next C partials (with
// the last chunk, the residual) all in flight before the first add, so a
// group costs a few memory round trips, not one per partial; the sum follows
// the fixed order P_0 + ... + P_{t-1} + R in fp32 and the row stays in
// registers.  Mean, then the biased variance of (x - mean), each a
// fixed-order block sum (lane swaps within each wave, then the waves' sums in
// order); y = (x - mean) * rsqrt(var + eps) * gamma + beta.  HBM-bound: t
// partials and the residual read, x and y written.
// ---------------------------------------------------------------------------
namespace {

template <int Ctrl>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), Ctrl, 0xf, 0xf, false));
}

// Sum of v over the wave's 64 lanes, the same bits in every lane: within each
// 16-lane row by DPP rotations (8, 4) and quad permutations (pairs 2 apart,
// then 1 apart), then across rows by a permlane16 and a permlane32 swap.
// Each step adds two lanes' values that the partner lane adds too, so all
// lanes agree bit for bit; no LDS round trip (the xor shuffles this replaces
// were six ds_bpermute waits per sum).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0x128>(v);  // row_ror:8
  v += dpp_mov<0x124>(v);  // row_ror:4
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  const auto a =
      __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b =
      __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float block_sum(float v, float* red, int nw) {
  v = wave_sum(v);
  __syncthreads();  // red[] free (a previous sum's readers are done)
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = red[0];
  for (int w = 1; w < nw; ++w) s += red[w];
  return s;
}

template <int DT>
__device__ __forceinline__ void store8_nt(void* base, int64_t g, const float* v) {
  if (DT == DT_BF16) {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = f2bf(v[2 * k]) | (f2bf(v[2 * k + 1]) << 16);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(base) + g);
  } else {
    f32x4* p = reinterpret_cast<f32x4*>(base) + 2 * g;
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, p);
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, p + 1);
  }
}

// The residual's group, its element type chosen at run time (uniform).
__device__ __forceinline__ Raw8 rawload8_dyn(const void* base, int dt, int64_t g) {
  return dt == DT_BF16 ? rawload8<DT_BF16>(base, g) : rawload8<DT_F32>(base, g);
}
__device__ __forceinline__ void add8_dyn(const Raw8& r, int dt, float* acc) {
  if (dt == DT_BF16)
    add8<DT_BF16>(r, acc);
  else
    add8<DT_F32>(r, acc);
}

// At most 512 threads (8 waves) per row: with the registers of up to three
// groups per thread two rows' workgroups share a CU, so one row's loads
// overlap the other's reductions and stores (a 768-thread row at 87
// registers left one row per CU: 4.85 -> 5.43 TB/s at 12288 columns, 4.47
// -> 5.31 at 8192).
template <int G>
struct LnThreads {
  static constexpr int value = 512;
};

template <int PDT, int C, int G>
__global__ void __launch_bounds__(LnThreads<G>::value)
reduce_ln_kernel(ReducePtrs ptrs, int t, const void* R, int rdt, void* xout, int xdt,
                 void* yout, int ydt, const float* gamma, const float* beta, float eps,
                 int64_t rows, int cols) {
  __shared__ float red[16];
  const int ng = cols / 8;  // 8-element groups per row
  const int nt = blockDim.x, nw = nt >> 6;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const int64_t g0 = row * ng;
    // slot j: group threadIdx.x + nt*j of the row, if it exists (a missing
    // one re-reads the row's first group and is neither summed nor stored)
    auto ok = [&](int j) { return (int)threadIdx.x + nt * j < ng; };
    auto gi = [&](int j) { return g0 + (ok(j) ? (int)threadIdx.x + nt * j : 0); };
    // Slot by slot (a row spans 512 threads at most, so a workgroup has
    // 8 KB x (C + 2) of loads in flight per chunk even one slot at a
    // time), chunk by chunk: partial 0, partials 1..C and, with the last
    // chunk, the residual are loaded before the first add.
    float v[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      {
        const bool last = 1 + C >= t;
        Raw8 pv[C], rr;
        const Raw8 r0 = rawload8<PDT>(ptrs.p[0], gi(j));
#pragma unroll
        for (int u = 0; u < C; ++u) pv[u] = rawload8<PDT>(ptrs.p[1 + u < t ? 1 + u : t - 1], gi(j));
        if (R != nullptr && last) rr = rawload8_dyn(R, rdt, gi(j));
        unpack8<PDT>(r0, v[j]);
#pragma unroll
        for (int u = 0; u < C; ++u)
          if (1 + u < t) add8<PDT>(pv[u], v[j]);
        if (R != nullptr && last) add8_dyn(rr, rdt, v[j]);
      }
      for (int i0 = 1 + C; i0 < t; i0 += C) {
        const bool last = i0 + C >= t;
        Raw8 pv[C], rr;
#pragma unroll
        for (int u = 0; u < C; ++u) pv[u] = rawload8<PDT>(ptrs.p[i0 + u < t ? i0 + u : t - 1], gi(j));
        if (R != nullptr && last) rr = rawload8_dyn(R, rdt, gi(j));
#pragma unroll
        for (int u = 0; u < C; ++u)
          if (i0 + u < t) add8<PDT>(pv[u], v[j]);
        if (R != nullptr && last) add8_dyn(rr, rdt, v[j]);
      }
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (ok(j))
#pragma unroll
        for (int e = 0; e < 8; ++e) s += v[j][e];
    const float mean = block_sum(s, red, nw) / (float)cols;
    float q = 0.0f;
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (ok(j))
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = v[j][e] - mean;
          q = __builtin_fmaf(d, d, q);
        }
    const float var = block_sum(q, red, nw) / (float)cols;
    const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (!ok(j)) continue;
      const int64_t g = gi(j);
      if (xout != nullptr) {
        if (xdt == DT_BF16)
          store8_nt<DT_BF16>(xout, g, v[j]);
        else
          store8_nt<DT_F32>(xout, g, v[j]);
      }
      const int c8 = (int)(g - g0);  // group within the row
      float gm[8], bt[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        gm[e] = 1.0f;
        bt[e] = 0.0f;
      }
      if (gamma != nullptr) {
        const f32x4* pg = reinterpret_cast<const f32x4*>(gamma) + 2 * c8;
        const f32x4 a = pg[0], b = pg[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gm[e] = a[e];
          gm[4 + e] = b[e];
        }
      }
      if (beta != nullptr) {
        const f32x4* pb = reinterpret_cast<const f32x4*>(beta) + 2 * c8;
        const f32x4 a = pb[0], b = pb[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bt[e] = a[e];
          bt[4 + e] = b[e];
        }
      }
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = __builtin_fmaf((v[j][e] - mean) * rstd, gm[e], bt[e]);
      if (ydt == DT_BF16)
        store8_nt<DT_BF16>(yout, g, y);
      else
        store8_nt<DT_F32>(yout, g, y);
    }
  }
}

template <int PDT, int C, int G>
hipError_t launch_ln(const ReducePtrs& ptrs, int t, const void* R, int rdt, void* xout, int xdt,
                     void* yout, int ydt, const float* gamma, const float* beta, float eps,
                     int64_t rows, int cols, hipStream_t s) {
  const int ng = cols / 8;
  const int nt = 64 * ((ng + 64 * G - 1) / (64 * G));  // threads per row: G groups each
  const int64_t blocks = rows < ((int64_t)1 << 24) - 1 ? rows : ((int64_t)1 << 24) - 1;
  hipLaunchKernelGGL((reduce_ln_kernel<PDT, C, G>), dim3((unsigned)blocks), dim3(nt), 0, s, ptrs,
                     t, R, rdt, xout, xdt, yout, ydt, gamma, beta, eps, rows, cols);
  return hipGetLastError();
}

// Groups per thread: the fewest of 1, 2, 3, 4, 6, 8 that keep a row within
// 512 threads.
template <int PDT, int C>
hipError_t launch_ln_g(const ReducePtrs& ptrs, int t, const void* R, int rdt, void* xout,
                       int xdt, void* yout, int ydt, const float* gamma, const float* beta,
                       float eps, int64_t rows, int cols, hipStream_t s) {
#define TP_LN_G(G) \
  launch_ln<PDT, C, G>(ptrs, t, R, rdt, xout, xdt, yout, ydt, gamma, beta, eps, rows, cols, s)
  const int ng = cols / 8;
  if (ng <= 512) return TP_LN_G(1);
  if (ng <= 1024) return TP_LN_G(2);
  if (ng <= 1536) return TP_LN_G(3);
  if (ng <= 2048) return TP_LN_G(4);
  if (ng <= 3072) return TP_LN_G(6);
  if (ng <= 4096) return TP_LN_G(8);
  return hipErrorInvalidValue;
#undef TP_LN_G
}

// Chunk size as for the reduce: t-1 for t <= 8 (no duplicate loads), 8 beyond.
template <int PDT>
hipError_t launch_ln_c(const ReducePtrs& ptrs, int t, const void* R, int rdt, void* xout,
                       int xdt, void* yout, int ydt, const float* gamma, const float* beta,
                       float eps, int64_t rows, int cols, hipStream_t s) {
#define TP_LN_ARGS ptrs, t, R, rdt, xout, xdt, yout, ydt, gamma, beta, eps, rows, cols, s
  switch (t) {
    case 1:
    case 2: return launch_ln_g<PDT, 1>(TP_LN_ARGS);
    case 3: return launch_ln_g<PDT, 2>(TP_LN_ARGS);
    case 4: return launch_ln_g<PDT, 3>(TP_LN_ARGS);
    case 5: return launch_ln_g<PDT, 4>(TP_LN_ARGS);
    case 6: return launch_ln_g<PDT, 5>(TP_LN_ARGS);
    case 7: return launch_ln_g<PDT, 6>(TP_LN_ARGS);
    case 8: return launch_ln_g<PDT, 7>(TP_LN_ARGS);
    default: return launch_ln_g<PDT, 8>(TP_LN_ARGS);
  }
#undef TP_LN_ARGS
}

}  // namespace

hipError_t reduce_layernorm(const ReducePtrs& ptrs, int t, int pdt, const void* R, int rdt,
                            void* xout, int xdt, void* yout, int ydt, const float* gamma,
                            const float* beta, float eps, int64_t rows, int cols,
                            hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (cols % 8 || cols > kLnMaxCols) return hipErrorInvalidValue;
  return pdt == DT_BF16 ? launch_ln_c<DT_BF16>(ptrs, t, R, rdt, xout, xdt, yout, ydt, gamma,
                                               beta, eps, rows, cols, s)
                        : launch_ln_c<DT_F32>(ptrs, t, R, rdt, xout, xdt, yout, ydt, gamma,
                                              beta, eps, rows, cols, s);
}

}  // namespace tp
