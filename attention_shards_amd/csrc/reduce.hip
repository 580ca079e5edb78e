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
  int64_t blocks = (ngroups + 255) / 256;
  if (blocks > (int64_t)1 << 30) blocks = (int64_t)1 << 30;
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

}  // namespace tp
