// Per-head softmax attention over a GPU's local heads (heads never talk to
// each other: page "Tensor Parallelism > Combining Column and Row
// Parallelism", the attention paragraphs).  Flash-style: one workgroup owns
// 64 queries of one (sequence, head) and streams 64-key tiles of K and V
// through LDS with an online softmax, so the score matrix never reaches HBM.
//
// Precision: Q and K arrive as bf16 hi/lo pairs, V as an fp16 hi/lo pair.
// Scores use three bf16 MFMA passes (Khi.Qhi + Khi.Qlo + Klo.Qhi, ~16
// significant bits); the softmax runs in fp32 with exp2; probabilities are
// rounded to fp16 (values in [0, 1], 11 significant bits) and the running
// denominator sums exactly those rounded values; P.V uses two fp16 MFMA
// passes (P.Vhi + P.Vlo).  O is written as a bf16 hi/lo pair, so the output
// projection sees it with ~16 significant bits.  Causal attention over short
// prefixes makes max|Y|/RMS(Y) large (row 0 is v_0 itself), which is what
// rules out single bf16 roundings of P and O here.
//
// Layout per wave (16 queries, v_mfma_f32_16x16x32_bf16):
//   * scores are computed transposed, S^T = K Q^T: A = K rows (keys),
//     B = Q (queries), so each lane ends up owning one query (lane % 16) and
//     four keys per 16-key block.  K rows are fed in the order that gives
//     lane group g = lane/16 the keys 8g..8g+7 of each 32-key chunk, which is
//     exactly the B operand of the next product;
//   * O^T = V^T P^T: A = V^T rows (head dims, keys contiguous in the V^T
//     workspace), B = P^T straight from the score registers.  The query of
//     every accumulator is again lane % 16, so softmax rescales are lane-local
//     and only the row max needs two cross-lane exchanges.
#include "internal.h"

namespace tp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;   // head dim
constexpr int QB = 64;   // queries per workgroup (4 waves x 16)
constexpr int KT = 64;   // keys per tile
constexpr int K_ROW = D * 2;    // 256-byte K rows (16 chunks)
constexpr int V_ROW = KT * 2;   // 128-byte V^T rows (8 chunks)
constexpr int TILE = KT * D * 2;  // 16 KiB per array

__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// K tile chunk swizzle: the 16 rows read together are
// {8a + 4b + c : a, c in 0..3} (+const); map them to 16 distinct chunks.
__device__ __forceinline__ int kswz(int r) { return (r & 3) | (((r >> 3) & 3) << 2); }
// V^T tile chunk swizzle (8 chunks per row; 16 consecutive rows read together).
__device__ __forceinline__ int vswz(int r) { return (r ^ (r >> 3)) & 7; }

__global__ void __launch_bounds__(256)
attn_fwd_kernel(QkvOut q, int batch, int causal, uint16_t* __restrict__ O,
                int nq, float scale_log2) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * TILE];
  uint8_t* sKh = smem;
  uint8_t* sKl = smem + TILE;
  uint8_t* sVh = smem + 2 * TILE;
  uint8_t* sVl = smem + 3 * TILE;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nbh = batch * q.nl;
  const int qb = nq - 1 - (int)(blockIdx.x / nbh);  // longest causal rows first
  const int bh = blockIdx.x % nbh;
  const int b = bh / q.nl, head = bh - b * q.nl;
  const int S = q.seq, Sp = q.seq_pad;
  const int64_t hoff = (int64_t)bh * Sp * D;
  const uint16_t* Qh = q.q_hi + hoff;
  const uint16_t* Ql = q.q_lo + hoff;
  const uint16_t* Kh = q.k_hi + hoff;
  const uint16_t* Kl = q.k_lo + hoff;
  const uint16_t* Vh = q.vt_hi + hoff;
  const uint16_t* Vl = q.vt_lo + hoff;

  const int g = lane >> 4;          // lane group
  const int myq = qb * QB + wave * 16 + (lane & 15);

  // Q as the B operand: query myq, head dims dc*32 + 8g .. +7.
  bf16x8 qh[4], ql[4];
#pragma unroll
  for (int dc = 0; dc < 4; ++dc) {
    if (myq < S) {
      qh[dc] = *reinterpret_cast<const bf16x8*>(Qh + (int64_t)myq * D + dc * 32 + 8 * g);
      ql[dc] = *reinterpret_cast<const bf16x8*>(Ql + (int64_t)myq * D + dc * 32 + 8 * g);
    } else {
      u32x4 z = {0, 0, 0, 0};
      qh[dc] = __builtin_bit_cast(bf16x8, z);
      ql[dc] = qh[dc];
    }
  }

  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{0, 0, 0, 0};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  const int n_kt = causal ? (qb + 1) : (S + KT - 1) / KT;
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * KT;
    __syncthreads();  // the previous tile is no longer read
    // K hi/lo: 64 rows x 16 chunks each; V^T hi/lo: 128 rows x 8 chunks each.
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = p * 256 + tid;
      const int r = idx >> 4, c = idx & 15;
      u32x4 vh = {0, 0, 0, 0}, vl = {0, 0, 0, 0};
      if (k0 + r < S) {
        vh = *reinterpret_cast<const u32x4*>(Kh + (int64_t)(k0 + r) * D + c * 8);
        vl = *reinterpret_cast<const u32x4*>(Kl + (int64_t)(k0 + r) * D + c * 8);
      }
      const int off = r * K_ROW + ((c ^ kswz(r)) << 4);
      *reinterpret_cast<u32x4*>(sKh + off) = vh;
      *reinterpret_cast<u32x4*>(sKl + off) = vl;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = p * 256 + tid;
      const int r = idx >> 3, c = idx & 7;
      const int key0 = k0 + c * 8;
      u32x4 vh = {0, 0, 0, 0}, vl = {0, 0, 0, 0};
      if (key0 < S) {
        vh = *reinterpret_cast<const u32x4*>(Vh + (int64_t)r * Sp + key0);
        vl = *reinterpret_cast<const u32x4*>(Vl + (int64_t)r * Sp + key0);
        if (key0 + 8 > S) {  // ragged tail: zero the keys past the sequence
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int kk = key0 + 2 * w;
            const uint32_t keep = (kk + 1 < S) ? 0xFFFFFFFFu : (kk < S ? 0x0000FFFFu : 0u);
            vh[w] &= keep;
            vl[w] &= keep;
          }
        }
      }
      const int off = r * V_ROW + ((c ^ vswz(r)) << 4);
      *reinterpret_cast<u32x4*>(sVh + off) = vh;
      *reinterpret_cast<u32x4*>(sVl + off) = vl;
    }
    __syncthreads();

    // ---- scores S^T for four 16-key blocks (chunk kc, half hb) ----
    f32x4 s[2][2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int i = lane & 15;
        const int krow = kc * 32 + 8 * (i >> 2) + 4 * hb + (i & 3);
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
          const int ch = dc * 4 + g;
          const int off = krow * K_ROW + ((ch ^ kswz(krow)) << 4);
          const bf16x8 kh = *reinterpret_cast<const bf16x8*>(sKh + off);
          const bf16x8 kl = *reinterpret_cast<const bf16x8*>(sKl + off);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh[dc], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, ql[dc], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qh[dc], acc, 0, 0, 0);
        }
        s[kc][hb] = acc;
      }

    // ---- online softmax; lane owns query myq and keys k0+kc*32+8g+4hb+e ----
    float mt = -__builtin_inff();
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = k0 + kc * 32 + 8 * g + 4 * hb + e;
          float v = s[kc][hb][e] * scale_log2;
          if (key >= S || (causal && key > myq)) v = -__builtin_inff();
          s[kc][hb][e] = v;
          mt = fmaxf(mt, v);
        }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -__builtin_inff()) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.0f;
    f16x8 pb[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const _Float16 p = (_Float16)__builtin_amdgcn_exp2f(s[kc][hb][e] - m_use);
          psum += (float)p;
          pb[kc][hb * 4 + e] = p;
        }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] *= alpha;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int drow = db * 16 + (lane & 15);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int ch = kc * 4 + g;
        const int off = drow * V_ROW + ((ch ^ vswz(drow)) << 4);
        const f16x8 vh = *reinterpret_cast<const f16x8*>(sVh + off);
        const f16x8 vl = *reinterpret_cast<const f16x8*>(sVl + off);
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, pb[kc], o[db], 0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl, pb[kc], o[db], 0, 0, 0);
      }
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (myq < S) {
    const float inv = 1.0f / l_tot;
    const int hd = q.nl * D;
    uint16_t* orow = O + ((int64_t)b * S + myq) * (2 * hd) + head * D;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      // O^T layout: lane owns head dims db*16 + 4g + e, e = 0..3
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = o[db][e] * inv;
        hi[e] = f2bf(v);
        lo[e] = f2bf(v - __uint_as_float(hi[e] << 16));
      }
      *reinterpret_cast<uint2*>(orow + db * 16 + 4 * g) =
          uint2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
      *reinterpret_cast<uint2*>(orow + hd + db * 16 + 4 * g) =
          uint2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
    }
  }
}

}  // namespace

hipError_t attention_fwd(const QkvOut& q, int batch, bool causal, uint16_t* O,
                         hipStream_t s) {
  if (batch == 0 || q.seq == 0 || q.nl == 0) return hipSuccess;
  const int nq = (q.seq + QB - 1) / QB;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)q.d);
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(nq * batch * q.nl), dim3(256), 0, s,
                     q, batch, causal ? 1 : 0, O, nq, scale_log2);
  return hipGetLastError();
}

}  // namespace tp
