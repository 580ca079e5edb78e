// Sum of the t shard partials plus the residual, in HBM on one GPU:
//     out = ((P_0 + P_1) + ... + P_{t-1}) + R
// This is the arithmetic of the all-reduce of FFN step 3 followed by the
// residual add of the closing paragraph (page "Tensor Parallelism >
// Combining Column and Row Parallelism"), without any transfer between GPUs.
//
// Pure streaming, HBM-bound: each thread owns runs of 8 elements (16-byte
// bf16 vectors, 2 x 16-byte fp32 vectors), loads the same run of every
// partial before adding (several loads in flight), accumulates in fp32 in
// the fixed order above and rounds once.  Inputs are read with non-temporal
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

template <int PDT, int RDT, int ODT>
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
    float acc[8];
    load8<PDT>(ptrs.p[0], gi, acc);
    int i = 1;
    // four partials' loads in flight before their adds
    for (; i + 4 <= t; i += 4) {
      float v0[8], v1[8], v2[8], v3[8];
      load8<PDT>(ptrs.p[i], gi, v0);
      load8<PDT>(ptrs.p[i + 1], gi, v1);
      load8<PDT>(ptrs.p[i + 2], gi, v2);
      load8<PDT>(ptrs.p[i + 3], gi, v3);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = (((acc[k] + v0[k]) + v1[k]) + v2[k]) + v3[k];
    }
    for (; i < t; ++i) {
      float v[8];
      load8<PDT>(ptrs.p[i], gi, v);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] += v[k];
    }
    if (RDT != DT_NONE) {
      float r[8];
      load8<RDT>(R, gi, r);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] += r[k];
    }
    store8<ODT>(out, gi, acc);
  }
}

template <int PDT, int RDT, int ODT>
hipError_t launch(const ReducePtrs& ptrs, int t, const void* R, void* out,
                  int64_t n, hipStream_t s) {
  const int64_t ngroups = n / 8;
  int64_t blocks = (ngroups + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((reduce_kernel<PDT, RDT, ODT>), dim3((unsigned)blocks),
                     dim3(256), 0, s, ptrs, t, R, out, ngroups, (int)(n - ngroups * 8));
  return hipGetLastError();
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
