// Per-head softmax attention over a GPU's local heads (heads never talk to
// each other: page "Tensor Parallelism > Combining Column and Row
// Parallelism", the attention paragraphs).  Flash-style: a workgroup owns
// 128 queries of one (sequence, head) and streams 64-key tiles of K and V
// through LDS with an online softmax, so the score matrix never reaches HBM.
//
// Work split: a query block's key range is cut into chunks of `ch` tiles,
// one workgroup per (query block, chunk, head), longest query blocks first.
// With causal masking the key range grows with the query position, so
// whole-range workgroups would leave most CUs idle while the last query
// blocks finish; chunks keep every workgroup's work within `ch` tiles.  A
// query block with one chunk writes O directly; otherwise each chunk writes
// its unnormalised O, running max and denominator, and a second kernel
// merges the chunks (the usual rescale by exp2(m_c - max m)).
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
// Layout per wave (32 queries as two groups of 16, v_mfma_f32_16x16x32_bf16):
//   * scores are computed transposed, S^T = K Q^T: A = K rows (keys),
//     B = Q (queries), so each lane ends up owning one query (lane % 16) of
//     each group and four keys per 16-key block.  K rows are fed in the
//     order that gives lane group g = lane/16 the keys 8g..8g+7 of each
//     32-key chunk, which is exactly the B operand of the next product.
//     Each K fragment read from LDS feeds both query groups;
//   * O^T = V^T P^T: A = V^T rows (head dims, keys contiguous in the V^T
//     workspace), B = P^T straight from the score registers.  The query of
//     every accumulator is again lane % 16, so softmax rescales are lane-local
//     and only the row max needs two cross-lane exchanges.  Each V fragment
//     read feeds both query groups.
#include "internal.h"

namespace tp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;    // head dim
constexpr int QW = 32;    // queries per wave (two groups of 16)
constexpr int QB = 128;   // queries per workgroup (4 waves)
constexpr int KT = 64;    // keys per tile
constexpr int K_ROW = D * 2;      // 256-byte K rows (16 chunks)
constexpr int V_ROW = KT * 2;     // 128-byte V^T rows (8 chunks)
constexpr int TILE = KT * D * 2;  // 16 KiB per array
constexpr int TARGET_ITEMS = 1024;  // aim for about four workgroups per CU

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

__host__ __device__ inline int div_up(int a, int b) { return (a + b - 1) / b; }

// Key tiles a query block needs.
__host__ __device__ inline int ntile_of(int qb, int seq, int causal) {
  const int kend = causal ? (QB * (qb + 1) < seq ? QB * (qb + 1) : seq) : seq;
  return div_up(kend, KT);
}

__global__ void __launch_bounds__(256)
attn_fwd_kernel(QkvOut q, int causal, uint16_t* __restrict__ O, float* __restrict__ part,
                AttnSplit sp, float scale_log2) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * TILE];
  uint8_t* sKh = smem;
  uint8_t* sKl = smem + TILE;
  uint8_t* sVh = smem + 2 * TILE;
  uint8_t* sVl = smem + 3 * TILE;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = q.seq, Sp = q.seq_pad;
  // workgroup -> (query block qb, chunk c, sequence*head bh)
  int rem = blockIdx.x, qb = sp.nqb - 1, nc = 1;
  for (;; --qb) {
    nc = div_up(ntile_of(qb, S, causal), sp.ch);
    if (rem < nc * sp.nbh || qb == 0) break;
    rem -= nc * sp.nbh;
  }
  const int c = rem / sp.nbh, bh = rem - c * sp.nbh;
  const int b = bh / q.nl, head = bh - b * q.nl;
  const int ntile = ntile_of(qb, S, causal);
  const int kt0 = c * sp.ch;
  const int kt1 = kt0 + sp.ch < ntile ? kt0 + sp.ch : ntile;

  const int64_t hoff = (int64_t)bh * Sp * D;
  const uint16_t* Qh = q.q_hi + hoff;
  const uint16_t* Ql = q.q_lo + hoff;
  const uint16_t* Kh = q.k_hi + hoff;
  const uint16_t* Kl = q.k_lo + hoff;
  const uint16_t* Vh = q.vt_hi + hoff;
  const uint16_t* Vl = q.vt_lo + hoff;

  const int g = lane >> 4;  // lane group
  int myq[2];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) myq[qg] = qb * QB + wave * QW + qg * 16 + (lane & 15);

  // Q as the B operand: query myq, head dims dc*32 + 8g .. +7.
  bf16x8 qh[2][4], ql[2][4];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg)
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
      if (myq[qg] < S) {
        qh[qg][dc] = *reinterpret_cast<const bf16x8*>(Qh + (int64_t)myq[qg] * D + dc * 32 + 8 * g);
        ql[qg][dc] = *reinterpret_cast<const bf16x8*>(Ql + (int64_t)myq[qg] * D + dc * 32 + 8 * g);
      } else {
        const u32x4 z = {0, 0, 0, 0};
        qh[qg][dc] = __builtin_bit_cast(bf16x8, z);
        ql[qg][dc] = qh[qg][dc];
      }
    }

  f32x4 o[2][8];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg)
#pragma unroll
    for (int db = 0; db < 8; ++db) o[qg][db] = f32x4{0, 0, 0, 0};
  float m_run[2] = {-__builtin_inff(), -__builtin_inff()};
  float l_run[2] = {0.0f, 0.0f};

  // Tile loads go through registers one tile ahead: the global loads of
  // tile kt+1 are issued before tile kt's products and land in LDS after
  // them.  K hi/lo: 64 rows x 16 chunks each; V^T hi/lo: 128 rows x 8
  // chunks each; every thread moves 4 chunks of each array.
  u32x4 rkh[4], rkl[4], rvh[4], rvl[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = p * 256 + tid;
      const int r = idx >> 4, cc = idx & 15;
      rkh[p] = u32x4{0, 0, 0, 0};
      rkl[p] = rkh[p];
      if (k0 + r < S) {
        rkh[p] = *reinterpret_cast<const u32x4*>(Kh + (int64_t)(k0 + r) * D + cc * 8);
        rkl[p] = *reinterpret_cast<const u32x4*>(Kl + (int64_t)(k0 + r) * D + cc * 8);
      }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = p * 256 + tid;
      const int r = idx >> 3, cc = idx & 7;
      const int key0 = k0 + cc * 8;
      rvh[p] = u32x4{0, 0, 0, 0};
      rvl[p] = rvh[p];
      if (key0 < S) {
        rvh[p] = *reinterpret_cast<const u32x4*>(Vh + (int64_t)r * Sp + key0);
        rvl[p] = *reinterpret_cast<const u32x4*>(Vl + (int64_t)r * Sp + key0);
      }
    }
  };
  auto sstore = [&](int k0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = p * 256 + tid;
      const int r = idx >> 4, cc = idx & 15;
      const int off = r * K_ROW + ((cc ^ kswz(r)) << 4);
      *reinterpret_cast<u32x4*>(sKh + off) = rkh[p];
      *reinterpret_cast<u32x4*>(sKl + off) = rkl[p];
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = p * 256 + tid;
      const int r = idx >> 3, cc = idx & 7;
      const int key0 = k0 + cc * 8;
      u32x4 vh = rvh[p], vl = rvl[p];
      if (key0 < S && key0 + 8 > S) {  // ragged tail: zero the keys past the sequence
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int kk = key0 + 2 * w;
          const uint32_t keep = (kk + 1 < S) ? 0xFFFFFFFFu : (kk < S ? 0x0000FFFFu : 0u);
          vh[w] &= keep;
          vl[w] &= keep;
        }
      }
      const int off = r * V_ROW + ((cc ^ vswz(r)) << 4);
      *reinterpret_cast<u32x4*>(sVh + off) = vh;
      *reinterpret_cast<u32x4*>(sVl + off) = vl;
    }
  };

  gload(kt0 * KT);
  for (int kt = kt0; kt < kt1; ++kt) {
    const int k0 = kt * KT;
    __syncthreads();  // the previous tile is no longer read
    sstore(k0);
    __syncthreads();
    if (kt + 1 < kt1) gload(k0 + KT);

    // ---- scores S^T for four 16-key blocks (chunk kc, half hb) ----
    f32x4 s[2][2][2];  // [query group][kc][hb]
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int i = lane & 15;
        const int krow = kc * 32 + 8 * (i >> 2) + 4 * hb + (i & 3);
        f32x4 a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
          const int ch = dc * 4 + g;
          const int off = krow * K_ROW + ((ch ^ kswz(krow)) << 4);
          const bf16x8 kh = *reinterpret_cast<const bf16x8*>(sKh + off);
          const bf16x8 kl = *reinterpret_cast<const bf16x8*>(sKl + off);
          a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh[0][dc], a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh[1][dc], a1, 0, 0, 0);
          a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, ql[0][dc], a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, ql[1][dc], a1, 0, 0, 0);
          a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qh[0][dc], a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qh[1][dc], a1, 0, 0, 0);
        }
        s[0][kc][hb] = a0;
        s[1][kc][hb] = a1;
      }

    // ---- online softmax; lane owns query myq[qg] and keys
    //      k0 + kc*32 + 8g + 4hb + e ----
    f16x8 pb[2][2];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
      float mt = -__builtin_inff();
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = k0 + kc * 32 + 8 * g + 4 * hb + e;
            float v = s[qg][kc][hb][e] * scale_log2;
            if (key >= S || (causal && key > myq[qg])) v = -__builtin_inff();
            s[qg][kc][hb][e] = v;
            mt = fmaxf(mt, v);
          }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run[qg], mt);
      const float m_use = (m_new == -__builtin_inff()) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[qg] - m_use);
      float psum = 0.0f;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const _Float16 p = (_Float16)__builtin_amdgcn_exp2f(s[qg][kc][hb][e] - m_use);
            psum += (float)p;
            pb[qg][kc][hb * 4 + e] = p;
          }
      l_run[qg] = l_run[qg] * alpha + psum;
      m_run[qg] = m_new;
#pragma unroll
      for (int db = 0; db < 8; ++db) o[qg][db] *= alpha;
    }

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
        o[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, pb[0][kc], o[0][db], 0, 0, 0);
        o[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, pb[1][kc], o[1][db], 0, 0, 0);
        o[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl, pb[0][kc], o[0][db], 0, 0, 0);
        o[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl, pb[1][kc], o[1][db], 0, 0, 0);
      }
    }
  }

  const int hd = q.nl * D;
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    float l_tot = l_run[qg] + __shfl_xor(l_run[qg], 16);
    l_tot += __shfl_xor(l_tot, 32);
    // O^T layout: lane owns head dims db*16 + 4g + e, e = 0..3
    if (nc == 1) {
      if (myq[qg] < S) {
        const float inv = 1.0f / l_tot;
        uint16_t* orow = O + ((int64_t)b * S + myq[qg]) * (2 * hd) + head * D;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = o[qg][db][e] * inv;
            hi[e] = f2bf(v);
            lo[e] = f2bf(v - __uint_as_float(hi[e] << 16));
          }
          *reinterpret_cast<uint2*>(orow + db * 16 + 4 * g) =
              uint2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
          *reinterpret_cast<uint2*>(orow + hd + db * 16 + 4 * g) =
              uint2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
        }
      }
    } else {
      // this chunk's unnormalised O, running max and denominator
      const int qi = wave * QW + qg * 16 + (lane & 15);
      float* po = part + ((int64_t)blockIdx.x * QB + qi) * D;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        *reinterpret_cast<f32x4*>(po + db * 16 + 4 * g) = o[qg][db];
      if (g == 0) {
        float* ml = part + (int64_t)sp.n_items * QB * D + ((int64_t)blockIdx.x * QB + qi) * 2;
        ml[0] = m_run[qg];
        ml[1] = l_tot;
      }
    }
  }
}

// Merge of the chunks of query blocks split in more than one.  A thread
// owns 8 head dims of one query: (query block, sequence*head) is
// blockIdx.x / 8, and 8 workgroups of 256 threads cover its 128 queries x
// 16 dim groups.  The weights exp2(m_c - max m) need every chunk's m first;
// the O loads of all chunks are then issued before the first multiply-add.
constexpr int MAXC = 16;  // chunks merged per pass (more are merged in passes)

__global__ void __launch_bounds__(256)
attn_combine_kernel(QkvOut q, int causal, uint16_t* __restrict__ O,
                    const float* __restrict__ part, AttnSplit sp) {
  const int grp = blockIdx.x >> 3;
  const int qb = grp / sp.nbh, bh = grp - qb * sp.nbh;
  const int S = q.seq;
  const int nc = div_up(ntile_of(qb, S, causal), sp.ch);
  if (nc == 1) return;
  int base = 0;  // first workgroup of this query block
  for (int x = sp.nqb - 1; x > qb; --x) base += div_up(ntile_of(x, S, causal), sp.ch) * sp.nbh;
  const int t = (blockIdx.x & 7) * 256 + threadIdx.x;  // 0..2047
  const int qi = t >> 4, dg = t & 15;                   // query in block, 8-dim group
  const int myq = qb * QB + qi;
  if (myq >= S) return;
  const float* ml = part + (int64_t)sp.n_items * QB * D;
  float M = -__builtin_inff();
  for (int c = 0; c < nc; ++c) {
    const int item = base + c * sp.nbh + bh;
    M = fmaxf(M, ml[((int64_t)item * QB + qi) * 2]);
  }
  float L = 0.0f;
  f32x4 a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
  for (int c0 = 0; c0 < nc; c0 += MAXC) {
    f32x4 x0[MAXC], x1[MAXC];
    float w[MAXC];
#pragma unroll
    for (int u = 0; u < MAXC; ++u) {
      const int c = c0 + u < nc ? c0 + u : nc - 1;  // past the end: re-read, weight 0
      const int64_t row = (int64_t)(base + c * sp.nbh + bh) * QB + qi;
      const f32x4* po = reinterpret_cast<const f32x4*>(part + row * D + dg * 8);
      x0[u] = po[0];
      x1[u] = po[1];
      const float mc = ml[row * 2];
      w[u] = (c0 + u >= nc || mc == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mc - M);
      L += w[u] * ml[row * 2 + 1];
    }
#pragma unroll
    for (int u = 0; u < MAXC; ++u) {
      a0 += w[u] * x0[u];
      a1 += w[u] * x1[u];
    }
  }
  const float inv = 1.0f / L;
  const int b = bh / q.nl, head = bh - b * q.nl;
  const int hd = q.nl * D;
  uint16_t* orow = O + ((int64_t)b * S + myq) * (2 * hd) + head * D + dg * 8;
  uint32_t hi[8], lo[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = (e < 4 ? a0[e] : a1[e - 4]) * inv;
    hi[e] = f2bf(v);
    lo[e] = f2bf(v - __uint_as_float(hi[e] << 16));
  }
  *reinterpret_cast<u32x4*>(orow) = u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16),
                                          hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)};
  *reinterpret_cast<u32x4*>(orow + hd) = u32x4{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16),
                                               lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)};
}

}  // namespace

AttnSplit attn_split(int batch, int seq, int nl, bool causal) {
  AttnSplit sp;
  sp.nbh = batch * nl;
  sp.nqb = div_up(seq, QB);
  int64_t tiles = 0;
  for (int qb = 0; qb < sp.nqb; ++qb) tiles += ntile_of(qb, seq, causal ? 1 : 0);
  tiles *= sp.nbh;
  int64_t ch = (tiles + TARGET_ITEMS - 1) / TARGET_ITEMS;
  sp.ch = (int)(ch < 4 ? 4 : ch);
  int64_t items = 0;
  for (int qb = 0; qb < sp.nqb; ++qb) items += div_up(ntile_of(qb, seq, causal ? 1 : 0), sp.ch);
  sp.n_items = (int)(items * sp.nbh);
  return sp;
}

int64_t attn_partial_bytes(int batch, int seq, int nl) {
  int64_t items = 0;
  for (int c = 0; c < 2; ++c) {
    const AttnSplit sp = attn_split(batch, seq, nl, c != 0);
    if (sp.n_items > items) items = sp.n_items;
  }
  return items * QB * (D + 2) * 4;
}

hipError_t attention_fwd(const QkvOut& q, int batch, bool causal, uint16_t* O, float* part,
                         hipStream_t s) {
  if (batch == 0 || q.seq == 0 || q.nl == 0) return hipSuccess;
  const AttnSplit sp = attn_split(batch, q.seq, q.nl, causal);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)q.d);
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(sp.n_items), dim3(256), 0, s, q, causal ? 1 : 0, O,
                     part, sp, scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (sp.n_items == sp.nqb * sp.nbh) return hipSuccess;  // no query block was split
  hipLaunchKernelGGL(attn_combine_kernel, dim3(sp.nqb * sp.nbh * 8), dim3(256), 0, s, q,
                     causal ? 1 : 0, O, part, sp);
  return hipGetLastError();
}

}  // namespace tp
