// Per-head softmax attention over a GPU's local heads (heads never talk to
// each other: page "Tensor Parallelism > Combining Column and Row
// Parallelism", the attention paragraphs).  Flash-style: a workgroup owns
// a block of 128 or 256 queries of one (sequence, head) and streams 64-key
// tiles of K and V through LDS with an online softmax, so the score matrix
// never reaches HBM.
//
// Work split: a query block's key range is cut into chunks of `ch` tiles,
// one workgroup per (query block, chunk, head), longest query blocks first.
// With causal masking the key range grows with the query position, so
// whole-range workgroups would leave most CUs idle while the last query
// blocks finish; chunks keep every workgroup's work within `ch` tiles.  A
// query block with one chunk writes O directly; otherwise each chunk writes
// its unnormalised O, running max and denominator, and a second kernel
// merges the chunks (the usual rescale by exp2(m_c - max m)).  The host
// picks the block size (256 when a dispatch estimate says it is faster:
// long sequences or many heads) and the chunk size per shape.
//
// Precision: Q and K arrive as fp16 values (11 significant bits), V as an
// fp16 hi/lo pair.  Scores use one fp16 MFMA pass; the softmax runs in fp32
// with exp2; probabilities are rounded to fp16 (values in [0, 1], 11
// significant bits) and the running denominator sums exactly those rounded
// values; P.V uses two fp16 MFMA passes (P.Vhi + P.Vlo).  O is written as
// fp16 plus its residual in bf8 (e5m2), so the output projection sees it
// with ~14 significant bits (one fp16 pass and one bf8 pass of half the
// cost).  Causal attention over short prefixes makes max|Y|/RMS(Y) large
// (row 0 is v_0 itself), which is what rules out single roundings of V and
// O here (an emulation of these rounding points on the CPU chose the split).
// Q, K and V must lie within the fp16 range (|x| < 65504).
//
// Layout: a workgroup has 8 waves (two per SIMD, so one wave's LDS waits
// overlap the other's MFMAs) of one or two groups of 16 queries each; per
// 16-query group, with v_mfma_f32_16x16x32_f16:
//   * scores are computed transposed, S^T = K Q^T: A = K rows (keys),
//     B = Q (queries), so each lane ends up owning one query (lane % 16)
//     and four keys per 16-key block.  K rows are fed in the order that
//     gives lane group g = lane/16 the keys 8g..8g+7 of each 32-key chunk,
//     which is exactly the B operand of the next product;
//   * O^T = V^T P^T: A = V^T rows (head dims, keys contiguous in the V^T
//     workspace), B = P^T straight from the score registers.  The query of
//     every accumulator is again lane % 16, so softmax rescales are lane-local
//     and only the row max needs two cross-lane exchanges.
#include <functional>
#include <map>
#include <mutex>
#include <queue>
#include <tuple>
#include <utility>
#include <vector>

#include "internal.h"

namespace tp {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Maximum of x over lanes l, l^16, l^32 and l^48 (the four 16-lane rows of
// the wave), by two register swaps across the rows instead of LDS
// permutes: permlane32_swap pairs lane l with l^32, permlane16_swap with
// l^16; with the same register as both operands each returned half holds
// one side of every pair.
__device__ __forceinline__ float max_of_four_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;    // head dim
constexpr int NWAVE = 8;  // waves per workgroup: two per SIMD, so one wave's
                          // LDS waits overlap the other's MFMAs
constexpr int NT = NWAVE * 64;   // threads per workgroup
// Each wave holds NQG groups of 16 queries (NQG = 1 or 2), so a workgroup
// covers a query block of 128 or 256 queries; the larger block reuses each
// K and V^T fragment read from LDS for twice the queries.
constexpr int KT = 64;    // keys per tile
constexpr int K_ROW = D * 2;      // 256-byte K rows (16 chunks)
constexpr int V_ROW = KT * 2;     // 128-byte V^T rows (8 chunks)
constexpr int TILE = KT * D * 2;  // 16 KiB per array
constexpr int NARR = 3;           // arrays per key tile: K, V^T hi, V^T lo
constexpr int NBUF = 3;           // key tiles in LDS: one multiplied, two landing
constexpr int MAX_ITEMS = 4096;  // bounds the partial-result workspace

__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// K tile chunk swizzle: the 16 rows read together are
// {8a + 4b + c : a, c in 0..3} (+const); map them to 16 distinct chunks.
__device__ __forceinline__ int kswz(int r) { return (r & 3) | (((r >> 3) & 3) << 2); }
// V^T tile chunk swizzle (8 chunks per row; 16 consecutive rows read together):
// the row's low three bits.  Measured with the LDS bank-conflict counter, this
// reads the 16-row fragments without conflicts; folding in row bit 3 as well
// cost about 3.8 conflict cycles per 16-byte read.
__device__ __forceinline__ int vswz(int r) { return r & 7; }

__host__ __device__ inline int div_up(int a, int b) { return (a + b - 1) / b; }

constexpr int OOB = 0x7FFFFFF0;  // buffer size cap; reads past a buffer return 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > (int64_t)OOB ? OOB : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// Global -> LDS copy of 16 bytes per lane (buffer_load ... lds): lane l's
// bytes land at LDS address lds_base + 16*l.  Issued from inline assembly,
// with completion tracked by wait_vmcnt() (m0 is set here and used by
// nothing else in this file's kernels).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, int voffset,
                                      uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// O for the output projection, [rows][hd] (hd = heads * D): O_hi, fp16,
// K-blocked by 32 ([hd/32][rows][32]); after it O_lo, bf8, K-blocked by 64
// ([hd/64][rows][64 bytes]) with each 64-byte row piece permuted so that
// byte 32h + 8s + j holds column 16s + 8h + j (s = 0..3, h = 0..1,
// j = 0..7), the order in which the projection's lo product consumes it.
// Element (fp16) offset of O_hi[row][col]:
__device__ __forceinline__ int64_t ohi_at(int64_t row, int col, int64_t rows) {
  return ((int64_t)(col >> 5) * rows + row) * 32 + (col & 31);
}
// Byte offset of O_lo[row][col] from the start of O_lo; col..col+3
// (col % 4 == 0) are contiguous, and so are col..col+7 for col % 8 == 0.
__device__ __forceinline__ int64_t olo_at(int64_t row, int col, int64_t rows) {
  const int k = col & 63;
  return ((int64_t)(col >> 6) * rows + row) * 64 + (((k >> 3) & 1) << 5) + ((k >> 4) << 3) +
         (k & 7);
}
// O_hi = fp16(x) (nearest even), O_lo = bf8(x - O_hi) with the residual
// taken exactly by one fma (written out, so the rounding does not depend on
// the compiler's contraction choices); x = o * inv.  Four values: two fp16
// pairs and four bf8 bytes.
__device__ __forceinline__ void o_split4(const float* o, float inv, uint32_t* hi, uint32_t* lo8) {
  float r[4];
#pragma unroll
  for (int e = 0; e < 4; e += 2) {
    const _Float16 h0 = (_Float16)(o[e] * inv), h1 = (_Float16)(o[e + 1] * inv);
    r[e] = __builtin_fmaf(o[e], inv, -(float)h0);
    r[e + 1] = __builtin_fmaf(o[e + 1], inv, -(float)h1);
    hi[e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
  }
  int v = __builtin_amdgcn_cvt_pk_bf8_f32(r[0], r[1], 0, false);
  v = __builtin_amdgcn_cvt_pk_bf8_f32(r[2], r[3], v, true);
  *lo8 = (uint32_t)v;
}

// Key tiles query block qb (of QB queries) needs.
__host__ __device__ inline int ntile_of(int qb, int seq, int causal, int QB) {
  const int kend = causal ? (QB * (qb + 1) < seq ? QB * (qb + 1) : seq) : seq;
  return div_up(kend, KT);
}

template <int NQG>
__global__ void __launch_bounds__(NT)
attn_fwd_kernel(QkvOut q, int causal, uint16_t* __restrict__ O,
                float* __restrict__ part, AttnSplit sp, float scale_log2) {
  constexpr int QW = 16 * NQG;    // queries per wave
  constexpr int QB = NWAVE * QW;  // queries per workgroup
  // Three LDS buffers of K, V^T hi, V^T lo tiles (144 KB): one is read by
  // the products while the next two tiles land in the others.
  __shared__ __attribute__((aligned(16))) uint8_t smem[NBUF * NARR * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int S = q.seq, Sp = q.seq_pad;
  // workgroup -> (query block qb, chunk c, sequence*head bh)
  int rem = blockIdx.x, qb = sp.nqb - 1, nc = 1;
  for (;; --qb) {
    nc = div_up(ntile_of(qb, S, causal, QB), sp.ch);
    if (rem < nc * sp.nbh || qb == 0) break;
    rem -= nc * sp.nbh;
  }
  const int c = rem / sp.nbh, bh = rem - c * sp.nbh;
  const int b = bh / q.nl, head = bh - b * q.nl;
  const int ntile = ntile_of(qb, S, causal, QB);
  const int kt0 = c * sp.ch;
  const int kt1 = kt0 + sp.ch < ntile ? kt0 + sp.ch : ntile;

  const int64_t hoff = (int64_t)bh * Sp * D;
  const uint16_t* Qp = q.q + hoff;
  const uint16_t* Kp = q.k + hoff;
  const uint16_t* Vh = q.vt_hi + hoff;
  const uint16_t* Vl = q.vt_lo + hoff;

  const int g = lane >> 4;  // lane group
  int myq[NQG];
#pragma unroll
  for (int qg = 0; qg < NQG; ++qg) myq[qg] = qb * QB + wave * QW + qg * 16 + (lane & 15);

  // Q as the B operand: query myq, head dims dc*32 + 8g .. +7.  Buffer loads:
  // queries past the sequence read as zero, so no load waits on a select.
  f16x8 qf[NQG][4];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qp, (int64_t)S * D * 2);
#pragma unroll
    for (int qg = 0; qg < NQG; ++qg)
#pragma unroll
      for (int dc = 0; dc < 4; ++dc) {
        const int off = myq[qg] < S ? (myq[qg] * D + dc * 32 + 8 * g) * 2 : OOB;
        qf[qg][dc] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      }
  }

  f32x4 o[NQG][8];
#pragma unroll
  for (int qg = 0; qg < NQG; ++qg)
#pragma unroll
    for (int db = 0; db < 8; ++db) o[qg][db] = f32x4{0, 0, 0, 0};
  float m_run[NQG], l_run[NQG];
#pragma unroll
  for (int qg = 0; qg < NQG; ++qg) {
    m_run[qg] = -__builtin_inff();
    l_run[qg] = 0.0f;
  }

  // Tiles go from global memory straight into LDS (buffer loads that write
  // LDS): while tile kt is multiplied from one buffer, tiles kt+1 and kt+2
  // land in the other two.  Each 1 KiB DMA covers 4 K rows (256 B) or 8 V^T rows
  // (128 B); lane l writes bytes 16l..16l+15 of it, so the chunk swizzles
  // are applied to the global addresses.  K rows past the sequence fall
  // outside the buffer descriptor and read as zero; V^T columns past it are
  // zero in the workspace (see attention_fwd).
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  constexpr int NDW = 16 / NWAVE;  // DMAs per wave per array
  int k_off[NDW], v_off[NDW];
#pragma unroll
  for (int j = 0; j < NDW; ++j) {
    const int i = j * NWAVE + wave;  // 1 KiB block of the array
    const int rk = 4 * i + (lane >> 4), pk = lane & 15;
    k_off[j] = rk * K_ROW + ((pk ^ kswz(rk)) << 4);
    const int rv = 8 * i + (lane >> 3), pv = lane & 7;
    v_off[j] = rv * Sp * 2 + ((pv ^ vswz(rv)) << 4);
  }
  auto stage = [&](int k0, int buf) {
    const uint32_t base = lds0 + buf * NARR * TILE;
    const int64_t kbytes = (int64_t)(S - k0) * D * 2;
    const int64_t vbytes = ((int64_t)D * Sp - k0) * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kp + (int64_t)k0 * D, kbytes);
    const __amdgpu_buffer_rsrc_t rvh = make_rsrc(Vh + k0, vbytes);
    const __amdgpu_buffer_rsrc_t rvl = make_rsrc(Vl + k0, vbytes);
#pragma unroll
    for (int j = 0; j < NDW; ++j) {
      const uint32_t blk = (j * NWAVE + wave) * 1024;
      dma16(rk, k_off[j], base + blk);
      dma16(rvh, v_off[j], base + TILE + blk);
      dma16(rvl, v_off[j], base + 2 * TILE + blk);
    }
  };
  // This wave's DMAs per key tile; waiting until at most that many are in
  // flight leaves exactly the latest tile's loads outstanding.
  constexpr int TILE_DMAS = NARR * NDW;

  stage(kt0 * KT, 0);
  // The Q fragments came from ordinary loads, which the compiler tracks; the
  // tile DMAs and their waits are inline assembly it cannot see.  Reading the
  // fragments here makes it wait for them (and, loads completing in order,
  // for tile kt0) once, before the loop; otherwise it leaves their wait to
  // the loop's first MFMA and, not knowing how many loads follow them, waits
  // for all of them there, draining the prefetch of tile kt+2 on every tile.
#pragma unroll
  for (int qg = 0; qg < NQG; ++qg)
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) asm volatile("" ::"v"(qf[qg][dc]));
  wait_vmcnt<0>();
  if (kt0 + 1 < kt1) stage((kt0 + 1) * KT, 1);
  __syncthreads();
  for (int kt = kt0; kt < kt1; ++kt) {
    const int k0 = kt * KT;
    const int cur = (kt - kt0) % NBUF;
    // Tile kt+2 into the third buffer; its last reader, tile kt-1, finished
    // before the barrier that ended the previous step.
    const bool ahead2 = kt + 2 < kt1;
    if (ahead2) stage(k0 + 2 * KT, cur == 0 ? 2 : cur - 1);
    // Causal: a tile that starts after this wave's last query is masked for
    // all of its queries and changes neither their softmax state nor O, so
    // the wave only takes part in the tile's loads and its closing barrier.
    if (causal && k0 > qb * QB + wave * QW + QW - 1) {
      if (ahead2)
        wait_vmcnt<TILE_DMAS>();
      else
        wait_vmcnt<0>();
      __syncthreads();
      continue;
    }
    const uint8_t* const sK = smem + cur * NARR * TILE;
    const uint8_t* const sVh = sK + TILE;
    const uint8_t* const sVl = sK + 2 * TILE;

    // ---- scores S^T for four 16-key blocks (chunk kc, half hb) ----
    // The four K fragments of 32-dim slice dc+1 are read while slice dc's
    // MFMAs run (two register sets), and the MFMAs cycle over independent
    // accumulators, so neither LDS latency nor an MFMA result holds the
    // matrix pipe.
    f32x4 s[NQG][2][2];  // [query group][kc][hb]
#pragma unroll
    for (int qg = 0; qg < NQG; ++qg)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) s[qg][kc][hb] = f32x4{0, 0, 0, 0};
    f16x8 kf[2][2][2];  // [set][kc][hb]
    auto kread = [&](int set, int dc) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int i = lane & 15;
          const int krow = kc * 32 + 8 * (i >> 2) + 4 * hb + (i & 3);
          const int off = krow * K_ROW + (((dc * 4 + g) ^ kswz(krow)) << 4);
          kf[set][kc][hb] = *reinterpret_cast<const f16x8*>(sK + off);
        }
    };
    kread(0, 0);
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
      const int set = dc & 1;
      if (dc + 1 < 4) kread(set ^ 1, dc + 1);
      // keep the next reads ahead of this step's MFMAs (the compiler would
      // otherwise sink each read to just before its use and wait on it)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int qg = 0; qg < NQG; ++qg)
            s[qg][kc][hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[set][kc][hb], qf[qg][dc],
                                                                  s[qg][kc][hb], 0, 0, 0);
    }

    // V fragments of the first PV group, read during the softmax below.
    f16x8 vh[2][4], vl[2][4];  // [set][db within the group]
    auto vread = [&](int set, int grp) {  // grp = kc*2 + half of the head dims
      const int kc = grp >> 1;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int db = (grp & 1) * 4 + u;
        const int drow = db * 16 + (lane & 15);
        const int off = drow * V_ROW + (((kc * 4 + g) ^ vswz(drow)) << 4);
        vh[set][u] = *reinterpret_cast<const f16x8*>(sVh + off);
        vl[set][u] = *reinterpret_cast<const f16x8*>(sVl + off);
      }
    };
    vread(0, 0);

    // ---- online softmax; lane owns query myq[qg] and keys
    //      k0 + kc*32 + 8g + 4hb + e.  Only the last key tile (keys past the
    //      sequence) and tiles reaching past the wave's first query (causal)
    //      need the mask.  Scores stay unscaled; the scale goes into the
    //      exponent's multiply-add.  The O rescale is skipped when no query
    //      of the wave raised its running max (alpha == 1 everywhere). ----
    const bool mask_tile = (k0 + KT > S) || (causal && k0 + KT - 1 > qb * QB + wave * QW);
    f16x8 pb[NQG][2];
#pragma unroll
    for (int qg = 0; qg < NQG; ++qg) {
      float mt = -__builtin_inff();
      if (mask_tile) {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int key = k0 + kc * 32 + 8 * g + 4 * hb + e;
              if (key >= S || (causal && key > myq[qg])) s[qg][kc][hb][e] = -__builtin_inff();
              mt = fmaxf(mt, s[qg][kc][hb][e]);
            }
      } else {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int e = 0; e < 4; ++e) mt = fmaxf(mt, s[qg][kc][hb][e]);
      }
      mt = max_of_four_rows(mt);
      const float m_new = fmaxf(m_run[qg], mt * scale_log2);
      const float m_use = (m_new == -__builtin_inff()) ? 0.0f : m_new;
      // probabilities rounded to fp16 in pairs; the denominator adds exactly
      // those rounded values, two per packed dot product with (1, 1)
      float psum = 0.0f;
      const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const float pa = __builtin_amdgcn_exp2f(
                __builtin_fmaf(s[qg][kc][hb][e], scale_log2, -m_use));
            const float pc = __builtin_amdgcn_exp2f(
                __builtin_fmaf(s[qg][kc][hb][e + 1], scale_log2, -m_use));
            const f16x2 p2 = __builtin_convertvector(f32x2{pa, pc}, f16x2);
            psum = __builtin_amdgcn_fdot2(p2, ones, psum, false);
            pb[qg][kc][hb * 4 + e] = p2[0];
            pb[qg][kc][hb * 4 + e + 1] = p2[1];
          }
      if (__builtin_amdgcn_ballot_w64(m_new != m_run[qg]) != 0) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[qg] - m_use);
        l_run[qg] = l_run[qg] * alpha + psum;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[qg][db] *= alpha;
      } else {
        l_run[qg] += psum;
      }
      m_run[qg] = m_new;
    }

    // ---- O^T += V^T P^T ----
    // Four groups (key half kc x half of the head dims) of eight V
    // fragments; group grp+1 is read while group grp's 16 MFMAs run, which
    // cycle over 8 independent accumulators.
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int set = grp & 1, kc = grp >> 1;
      if (grp + 1 < 4) vread(set ^ 1, grp + 1);
      __builtin_amdgcn_sched_barrier(0);  // (as for the K fragments above)
#pragma unroll
      for (int pass = 0; pass < 2; ++pass)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int qg = 0; qg < NQG; ++qg) {
            const int db = (grp & 1) * 4 + u;
            o[qg][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pass ? vl[set][u] : vh[set][u],
                                                               pb[qg][kc], o[qg][db], 0, 0, 0);
          }
    }
    // tile kt+1 has landed (this wave's part of it; tile kt+2's may still
    // be in flight) ...
    if (ahead2)
      wait_vmcnt<TILE_DMAS>();
    else
      wait_vmcnt<0>();
    __syncthreads();  // ... everyone's; and tile kt is no longer read
  }

  const int hd = q.nl * D;
#pragma unroll
  for (int qg = 0; qg < NQG; ++qg) {
    float l_tot = l_run[qg] + __shfl_xor(l_run[qg], 16);
    l_tot += __shfl_xor(l_tot, 32);
    // O^T layout: lane owns head dims db*16 + 4g + e, e = 0..3
    if (nc == 1) {
      if (myq[qg] < S) {
        const float inv = 1.0f / l_tot;
        const int64_t orow = (int64_t)b * S + myq[qg], rows = (int64_t)(sp.nbh / q.nl) * S;
        uint8_t* const olo = reinterpret_cast<uint8_t*>(O) + rows * hd * 2;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          uint32_t hi[2], lo8;
          const float x[4] = {o[qg][db][0], o[qg][db][1], o[qg][db][2], o[qg][db][3]};
          o_split4(x, inv, hi, &lo8);
          const int col = head * D + db * 16 + 4 * g;
          *reinterpret_cast<uint2*>(O + ohi_at(orow, col, rows)) = uint2{hi[0], hi[1]};
          *reinterpret_cast<uint32_t*>(olo + olo_at(orow, col, rows)) = lo8;
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
// blockIdx.x / (qb/16), and qb/16 workgroups of 256 threads cover its qb
// queries x 16 dim groups.  The weights exp2(m_c - max m) need every chunk's
// m: when all chunks fit one pass, their O runs and (m, l) pairs are loaded
// together and the weights follow; otherwise the maxima are read first.
// MAXC chunks are merged per pass (more in several passes); the host picks
// the smallest of 4, 8, 16 that covers the largest chunk count, so a pass
// issues no more loads than it needs.
template <int MAXC>
__global__ void __launch_bounds__(256)
attn_combine_kernel(QkvOut q, int causal, uint16_t* __restrict__ O,
                    const float* __restrict__ part, AttnSplit sp) {
  const int QB = sp.qb, wpg = QB / 16;
  const int grp = blockIdx.x / wpg;
  const int qb = grp / sp.nbh, bh = grp - qb * sp.nbh;
  const int S = q.seq;
  const int nc = div_up(ntile_of(qb, S, causal, QB), sp.ch);
  if (nc == 1) return;
  int base = 0;  // first workgroup of this query block
  for (int x = sp.nqb - 1; x > qb; --x) base += div_up(ntile_of(x, S, causal, QB), sp.ch) * sp.nbh;
  const int t = (blockIdx.x - grp * wpg) * 256 + threadIdx.x;  // 0..16*QB-1
  const int qi = t >> 4, dg = t & 15;                           // query in block, 8-dim group
  const int myq = qb * QB + qi;
  if (myq >= S) return;
  const float* ml = part + (int64_t)sp.n_items * QB * D;
  // chunk c's row of partial results (O run, then max and denominator in ml)
  auto row_of = [&](int c) { return (int64_t)(base + c * sp.nbh + bh) * QB + qi; };
  // one chunk's contribution, in chunk order: L += w l_c, a += w O_c
  float L = 0.0f;
  f32x4 a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
  auto accumulate = [&](float w, float lc, const f32x4& x0, const f32x4& x1) {
    L = __builtin_fmaf(w, lc, L);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a0[e] = __builtin_fmaf(w, x0[e], a0[e]);
      a1[e] = __builtin_fmaf(w, x1[e], a1[e]);
    }
  };
  if (nc <= MAXC) {
    // One pass (the host sizes MAXC to the largest chunk count): every
    // chunk's O run, max and denominator are loaded together, then the
    // weights exp2(m_c - max m) follow from the loaded maxima.
    f32x4 x0[MAXC], x1[MAXC];
    float mc[MAXC], lc[MAXC];
#pragma unroll
    for (int u = 0; u < MAXC; ++u) {
      const int64_t row = row_of(u < nc ? u : nc - 1);  // past the end: re-read, weight 0
      const f32x4* po = reinterpret_cast<const f32x4*>(part + row * D + dg * 8);
      x0[u] = po[0];
      x1[u] = po[1];
      mc[u] = ml[row * 2];
      lc[u] = ml[row * 2 + 1];
    }
    float M = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < MAXC; ++u) M = fmaxf(M, mc[u]);
#pragma unroll
    for (int u = 0; u < MAXC; ++u) {
      const float w =
          (u >= nc || mc[u] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mc[u] - M);
      accumulate(w, lc[u], x0[u], x1[u]);
    }
  } else {
    // Several passes of MAXC chunks: the maxima first.
    float M = -__builtin_inff();
    for (int c = 0; c < nc; ++c) M = fmaxf(M, ml[row_of(c) * 2]);
    for (int c0 = 0; c0 < nc; c0 += MAXC) {
      f32x4 x0[MAXC], x1[MAXC];
      float mc[MAXC], lc[MAXC];
#pragma unroll
      for (int u = 0; u < MAXC; ++u) {
        const int64_t row = row_of(c0 + u < nc ? c0 + u : nc - 1);
        const f32x4* po = reinterpret_cast<const f32x4*>(part + row * D + dg * 8);
        x0[u] = po[0];
        x1[u] = po[1];
        mc[u] = ml[row * 2];
        lc[u] = ml[row * 2 + 1];
      }
#pragma unroll
      for (int u = 0; u < MAXC; ++u) {
        const float w = (c0 + u >= nc || mc[u] == -__builtin_inff())
                            ? 0.0f
                            : __builtin_amdgcn_exp2f(mc[u] - M);
        accumulate(w, lc[u], x0[u], x1[u]);
      }
    }
  }
  const float inv = 1.0f / L;
  const int b = bh / q.nl, head = bh - b * q.nl;
  const int hd = q.nl * D;
  const int64_t orow = (int64_t)b * S + myq, rows = (int64_t)(sp.nbh / q.nl) * S;
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = e < 4 ? a0[e] : a1[e - 4];
  uint32_t hi[4], lo8[2];  // split as in attn_fwd_kernel
  o_split4(x, inv, hi, &lo8[0]);
  o_split4(x + 4, inv, hi + 2, &lo8[1]);
  const int col = head * D + dg * 8;
  *reinterpret_cast<u32x4*>(O + ohi_at(orow, col, rows)) = u32x4{hi[0], hi[1], hi[2], hi[3]};
  *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(O) + rows * hd * 2 +
                            olo_at(orow, col, rows)) = uint2{lo8[0], lo8[1]};
}

// Zeroes V^T columns [seq, seq_pad) of every (sequence*head, dim) row, hi
// and lo: the probabilities of those keys are 0, but 0 times whatever the
// workspace held there need not be.
__global__ void __launch_bounds__(256)
vt_pad_zero_kernel(QkvOut q, int64_t rows) {
  const int pad = q.seq_pad - q.seq;
  const int64_t n = (int64_t)rows * pad;
  for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < n; k += (int64_t)gridDim.x * 256) {
    const int64_t r = k / pad;
    const int64_t at = r * q.seq_pad + q.seq + (k - r * pad);
    q.vt_hi[at] = 0;
    q.vt_lo[at] = 0;
  }
}

// Estimated time, in units of one 64-key tile of a 128-query workgroup, of
// the attention kernel with query blocks of QB queries and chunks of `ch`
// tiles: workgroups are dispatched in grid order (longest query blocks
// first) onto the device's compute units, one at a time each (the LDS holds one), and
// cost a start-up (Q load, first tile round trip, partial write) plus their
// tiles; splitting a query block adds MERGE_COST per split workgroup and the
// merge kernel's MERGE_LAUNCH.  Per-variant costs: 128-query blocks start up
// in 4 tile units; 256-query blocks in 5, and a 256-query tile costs 1.6 (it
// reads the same K and V^T fragments from LDS for twice the queries).
// Fitted to measured kernel times at 200-8192 tokens and 2-24 local heads
// (about 10% RMS error; the sign of the difference between the two variants
// right at every measured shape).
constexpr double MERGE_COST = 0.004;
constexpr double MERGE_LAUNCH = 2.0;
struct VariantCost {
  int qb;
  double item, tile;
};
constexpr VariantCost VAR128 = {128, 4.0, 1.0};
constexpr VariantCost VAR256 = {256, 5.0, 1.6};

double split_cost(const VariantCost& v, int nqb, int nbh, int seq, int causal, int ch,
                  int ncu) {
  std::priority_queue<double, std::vector<double>, std::greater<double>> cu;
  for (int k = 0; k < ncu; ++k) cu.push(0.0);
  double end = 0.0;
  int64_t split = 0;
  for (int qb = nqb - 1; qb >= 0; --qb) {
    const int nt = ntile_of(qb, seq, causal, v.qb);
    const int nc = div_up(nt, ch);
    if (nc > 1) split += (int64_t)nc * nbh;
    for (int c = 0; c < nc; ++c) {
      const int tiles = nt - c * ch < ch ? nt - c * ch : ch;
      for (int bh = 0; bh < nbh; ++bh) {
        const double t0 = cu.top();
        cu.pop();
        const double t1 = t0 + v.item + v.tile * tiles;
        cu.push(t1);
        if (t1 > end) end = t1;
      }
    }
  }
  return end + MERGE_COST * (double)split + (split ? MERGE_LAUNCH : 0.0);
}

int64_t count_items(int qbs, int nqb, int seq, int causal, int ch) {
  int64_t items = 0;
  for (int qb = 0; qb < nqb; ++qb) items += div_up(ntile_of(qb, seq, causal, qbs), ch);
  return items;
}

// Chunk size for one variant, and its estimated time.  The default aims at
// about 1024 workgroups with chunks of at least 4 tiles.  Small problems pay
// for that in workgroup start-ups: when the estimate above finds a chunk of
// at most 16 tiles (grid within MAX_ITEMS) at least 10% cheaper, that one is
// used instead (8 heads, 2048 causal tokens, 128-query blocks: 10 tiles, 272
// workgroups, 54 us vs 68 us).  Larger chunks are not searched: there the
// estimate is least reliable and measured times vary by up to 40% between
// neighbouring sizes.  The one exception is the unsplit key range (one
// workgroup per query block, nothing to merge), taken when its estimate is
// at least 10% below the chosen chunk's: with many query blocks per CU the
// longest-first order pairs long and short ranges evenly (8 heads, 8192
// causal tokens, 128-query blocks: shard 939 us vs 986 us; 4 x 2048 tokens,
// 24 heads, 256-query blocks: 2820 us vs 2882 us).
std::pair<int, double> choose_chunk(const VariantCost& v, int nqb, int nbh, int seq, int causal,
                                    int ncu) {
  int64_t tiles = 0;
  for (int qb = 0; qb < nqb; ++qb) tiles += ntile_of(qb, seq, causal, v.qb);
  tiles *= nbh;
  const int64_t dflt = (tiles + 1023) / 1024;
  int best = (int)(dflt < 4 ? 4 : dflt);
  const double base = split_cost(v, nqb, nbh, seq, causal, best, ncu);
  double est = base;
  const int max_nt = ntile_of(nqb - 1, seq, causal, v.qb);  // the longest key range
  if (count_items(v.qb, nqb, seq, causal, 16 < max_nt ? 16 : max_nt) * nbh <= MAX_ITEMS) {
    double best_cost = base;
    int pick = best;
    for (int ch = 1; ch <= 16 && ch <= max_nt; ++ch) {
      if (count_items(v.qb, nqb, seq, causal, ch) * nbh > MAX_ITEMS) continue;
      const double cost = split_cost(v, nqb, nbh, seq, causal, ch, ncu);
      if (cost < best_cost * 0.999) {
        best_cost = cost;
        pick = ch;
      }
    }
    if (best_cost <= 0.9 * base) {
      best = pick;
      est = best_cost;
    }
  }
  if (max_nt > best && count_items(v.qb, nqb, seq, causal, max_nt) * nbh <= MAX_ITEMS) {
    const double whole = split_cost(v, nqb, nbh, seq, causal, max_nt, ncu);
    if (whole <= 0.9 * est) {
      best = max_nt;
      est = whole;
    }
  }
  return {best, est};
}

// Query block size and chunk size: 256-query blocks when their estimate is
// at least 3% below the 128-query one (long sequences and many heads; short
// ones have too few 256-query blocks to fill the GPU).  Memoised per shape.
AttnSplit choose_split(int batch, int seq, int nl, int causal) {
  static std::mutex m;
  static std::map<std::tuple<int, int, int, int, int>, AttnSplit> memo;
  const int ncu = device_cu_count();
  const auto key = std::make_tuple(batch, seq, nl, causal, ncu);
  {
    std::lock_guard<std::mutex> lock(m);
    const auto it = memo.find(key);
    if (it != memo.end()) return it->second;
  }
  AttnSplit sp;
  sp.nbh = batch * nl;
  const int nqb128 = div_up(seq, 128), nqb256 = div_up(seq, 256);
  const auto c128 = choose_chunk(VAR128, nqb128, sp.nbh, seq, causal, ncu);
  const auto c256 = choose_chunk(VAR256, nqb256, sp.nbh, seq, causal, ncu);
  const bool big = c256.second <= 0.97 * c128.second;
  sp.qb = big ? 256 : 128;
  sp.nqb = big ? nqb256 : nqb128;
  sp.ch = big ? c256.first : c128.first;
  sp.n_items = (int)(count_items(sp.qb, sp.nqb, seq, causal, sp.ch) * sp.nbh);
  std::lock_guard<std::mutex> lock(m);
  if (memo.size() > 1024) memo.clear();
  memo[key] = sp;
  return sp;
}

}  // namespace

AttnSplit attn_split(int batch, int seq, int nl, bool causal) {
  return choose_split(batch, seq, nl, causal ? 1 : 0);
}

int64_t attn_partial_bytes(int batch, int seq, int nl) {
  int64_t bytes = 0;
  for (int c = 0; c < 2; ++c) {
    const AttnSplit sp = attn_split(batch, seq, nl, c != 0);
    const int64_t b = (int64_t)sp.n_items * sp.qb * (D + 2) * 4;
    if (b > bytes) bytes = b;
  }
  return bytes;
}

hipError_t attention_fwd(const QkvOut& q, int batch, bool causal, uint16_t* O, float* part,
                         hipStream_t s) {
  if (batch == 0 || q.seq == 0 || q.nl == 0) return hipSuccess;
  const AttnSplit sp = attn_split(batch, q.seq, q.nl, causal);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)q.d);
  if (q.seq_pad > q.seq) {
    const int64_t rows = (int64_t)sp.nbh * D;
    const int64_t n = (int64_t)rows * (q.seq_pad - q.seq);
    const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(vt_pad_zero_kernel, dim3(blocks), dim3(256), 0, s, q, rows);
    const hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  if (sp.qb == 256)
    hipLaunchKernelGGL(attn_fwd_kernel<2>, dim3(sp.n_items), dim3(NT), 0, s, q, causal ? 1 : 0,
                       O, part, sp, scale_log2);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<1>, dim3(sp.n_items), dim3(NT), 0, s, q, causal ? 1 : 0,
                       O, part, sp, scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (sp.n_items == sp.nqb * sp.nbh) return hipSuccess;  // no query block was split
  const int max_nc = div_up(ntile_of(sp.nqb - 1, q.seq, causal ? 1 : 0, sp.qb), sp.ch);
  const dim3 grid(sp.nqb * sp.nbh * (sp.qb / 16));
  if (max_nc <= 4)
    hipLaunchKernelGGL(attn_combine_kernel<4>, grid, dim3(256), 0, s, q, causal ? 1 : 0, O,
                       part, sp);
  else if (max_nc <= 8)
    hipLaunchKernelGGL(attn_combine_kernel<8>, grid, dim3(256), 0, s, q, causal ? 1 : 0, O,
                       part, sp);
  else
    hipLaunchKernelGGL(attn_combine_kernel<16>, grid, dim3(256), 0, s, q, causal ? 1 : 0, O,
                       part, sp);
  return hipGetLastError();
}

}  // namespace tp
