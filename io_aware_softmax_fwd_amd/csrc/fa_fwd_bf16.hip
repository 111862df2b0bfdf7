// bf16 attention forward on the gfx950 matrix cores.
//
// One workgroup owns a tile of query rows of one (batch, head) and streams the
// K/V tiles of that head through LDS; the scores and probabilities of a tile
// live only in registers and are merged into a running row max m, row sum l
// and an unnormalised fp32 accumulator, which is rescaled by exp(m_old-m_new)
// whenever the max grows and divided by l once at the end (aiqz.cc Flash
// Attention IO article, sections 分块Tiling策略 and 在线Softmax算法; cf-1.com
// FlashAttention write-up, section 4.3).  Queries are the outer loop and keys
// the inner one, so each query tile reads Q once and writes O once.
//
// Layout of the work inside a workgroup (4 waves of 64 lanes):
//   * each wave owns QB blocks of 32 query rows, so row statistics never
//     leave the wave;
//   * scores are produced transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: K (from LDS) is the A operand and Q (kept in
//     registers for the whole kernel) the B operand.  In the accumulator
//     layout lane l then holds one query (l % 32) and 16 keys of each 32-key
//     block, so the row max and row sum are in-lane reductions plus one swap
//     with lane l ^ 32;
//   * the output is accumulated transposed as well, O^T += V^T P^T: the
//     probabilities are used in place as the B operand (converted to bf16)
//     and V^T comes from LDS, where V is stored transposed with the keys of
//     each 16-key group permuted to match the accumulator layout, so each
//     lane fetches its 8 keys with one 16-byte LDS read.
// Products accumulate in fp32; the softmax arithmetic is fp32, done as
// exp2(s*c - m*c) with c = scale*log2(e) folded into one FMA.
#include <math.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeys = 64;                 // keys per K/V tile (Bc)
constexpr float kLog2e = 1.4426950408889634f;

// LDS rows are padded by 16 bytes so that the 8 lanes served together by a
// 16-byte read hit 8 distinct 16-byte bank groups.
template <int D> struct Lds {
  static constexpr int kStride = D + 8;         // bf16 elements per K row
  static constexpr int vStride = kKeys + 8;     // bf16 elements per V^T row
  static constexpr int kBytes = kKeys * kStride * 2;
  static constexpr int vBytes = D * vStride * 2;
  static constexpr int total = kBytes + vBytes;
};

// Position of key k (0..63 inside a tile) in a V^T row: inside each group of
// 16 keys, key (e%4) + 8*(e/4) + 4*h is stored at 8*h + e, which is the order
// in which the score accumulator hands its keys to the P.V product.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~15) + 8 * ((k >> 2) & 1) + 4 * ((k >> 3) & 1) + (k & 3);
}

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;   // round to nearest even
  return (unsigned)__builtin_bit_cast(unsigned short, a) |
         ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
}

template <int D, int QB, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
    const unsigned short* __restrict__ v, unsigned short* __restrict__ o,
    float* __restrict__ lse, int N, int BH, int n_qtiles, float scale) {
  constexpr int BR = 32 * QB * kWaves;   // query rows per workgroup
  constexpr int KS = D / 16;             // k-steps of the score product
  constexpr int DB = D / 32;             // 32-wide blocks of the head dim
  constexpr int KB = kKeys / 32;         // 32-key blocks per tile
  constexpr int PS = kKeys / 16;         // k-steps of the P.V product

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned short* Ks = reinterpret_cast<unsigned short*>(smem);
  unsigned short* Vt = reinterpret_cast<unsigned short*>(smem + Lds<D>::kBytes);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // Heaviest query tiles first (causal work grows with the tile index); heads
  // vary fastest so that, with B*H a multiple of 8, all tiles of one head
  // land on the same XCD and share its L2.
  const int bh = blockIdx.x % BH;
  const int qt = n_qtiles - 1 - (int)(blockIdx.x / BH);
  const int q0 = qt * BR;
  const int qw = q0 + wave * 32 * QB;    // first query row of this wave
  const int64_t head = (int64_t)bh * N * D;
  const float c = scale * kLog2e;

  // ---- Q fragments: B operand of S^T = K Q^T, resident for the whole loop.
  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qw + 32 * qb + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qi < N)
        raw = *reinterpret_cast<const u32x4*>(q + head + (int64_t)qi * D + 16 * ks + 8 * hl);
      qf[qb][ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x16 acc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][db][r] = 0.f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m_run[qb] = -INFINITY; l_run[qb] = 0.f; }

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int n_tiles = (kv_end + kKeys - 1) / kKeys;

  for (int j = 0; j < n_tiles; ++j) {
    const int k0 = j * kKeys;
    __syncthreads();   // every wave is done with the previous tile

    // ---- K tile -> LDS, row-major.  16-byte loads, consecutive lanes walk
    // along a row, so every wave reads whole rows.
    constexpr int KCH = kKeys * D / 8 / kThreads;   // 16-byte chunks per thread
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int e = (u * kThreads + tid) * 8;
      const int r = e / D, col = e % D;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (k0 + r < N) raw = *reinterpret_cast<const u32x4*>(k + head + (int64_t)(k0 + r) * D + col);
      *reinterpret_cast<u32x4*>(Ks + r * Lds<D>::kStride + col) = raw;
    }
    // ---- V tile -> LDS transposed.  A thread loads KPT consecutive keys of
    // 8 dims and writes, for each dim, its keys as one contiguous run.
    constexpr int DG = D / 8;                       // 8-dim groups per row
    constexpr int KPT = kKeys * DG / kThreads;      // keys per thread (2 or 4)
    {
      const int dg = tid % DG;
      const int kg = tid / DG;
      u32x4 raw[KPT];
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int key = k0 + kg * KPT + i;
        raw[i] = u32x4{0u, 0u, 0u, 0u};
        if (key < N) raw[i] = *reinterpret_cast<const u32x4*>(v + head + (int64_t)key * D + 8 * dg);
      }
      const int pos = vt_pos(kg * KPT);
#pragma unroll
      for (int c2 = 0; c2 < 8; ++c2) {
        unsigned w[KPT / 2];
#pragma unroll
        for (int i = 0; i < KPT; i += 2) {
          const unsigned a = raw[i][c2 >> 1], b = raw[i + 1][c2 >> 1];
          w[i / 2] = (c2 & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        unsigned short* dst = Vt + (8 * dg + c2) * Lds<D>::vStride + pos;
        if constexpr (KPT == 4)
          *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
        else
          *reinterpret_cast<unsigned*>(dst) = w[0];
      }
    }
    __syncthreads();

    // Causal: a wave whose last query precedes the tile's first key has
    // nothing to do here (its barrier participation stays unconditional).
    if (CAUSAL && k0 > qw + 32 * QB - 1) continue;

    // ---- S^T = K_j Q^T on the matrix cores.
    f32x16 s[QB][KB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kf = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(Ks + (32 * kb + l32) * Lds<D>::kStride + 16 * ks + 8 * hl));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ks], s[qb][kb], 0, 0, 0);
      }
    }

    // ---- mask: keys past N (last tile) and, when causal, keys after the query.
    const bool need_mask = (k0 + kKeys > N) || (CAUSAL && k0 + kKeys - 1 > qw);
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qi = qw + 32 * qb + l32;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + (r & 3) + 8 * (r >> 2) + 4 * hl;
            if (key >= N || (CAUSAL && key > qi)) s[qb][kb][r] = -INFINITY;
          }
      }
    }

    // ---- online softmax, per query block.
    bf16x8 pf[QB][PS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));          // the other 32 keys of the tile
      const float m_new = fmaxf(m_run[qb], mx);
      const float mc = m_new * c;
      const float alpha = exp2f(m_run[qb] * c - mc);   // 0 while m_run = -inf
      // Rescale the accumulator only if some row of the wave raised its max.
      if (__any(m_new != m_run[qb])) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
      }
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float p0 = exp2f(fmaf(s[qb][kb][8 * half + e], c, -mc));
            const float p1 = exp2f(fmaf(s[qb][kb][8 * half + e + 1], c, -mc));
            psum += p0 + p1;
            w[e / 2] = pack_bf16x2(p0, p1);
          }
          pf[qb][2 * kb + half] = __builtin_bit_cast(bf16x8, w);
        }
      }
      l_run[qb] = l_run[qb] * alpha + psum;
      m_run[qb] = m_new;
    }

    // ---- O^T += V_j^T P^T on the matrix cores.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) {
        const bf16x8 vf = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(Vt + (32 * db + l32) * Lds<D>::vStride + 16 * ps + 8 * hl));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][ps], acc[qb][db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O = acc / l in bf16, LSE = scale*m + ln(l).
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qw + 32 * qb + l32;
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
    if (qi < N) {
      const float inv = 1.f / l_tot;
      unsigned short* orow = o + head + (int64_t)qi * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dim = 32 * db + 8 * g + 4 * hl;
          const u32x2 w = {pack_bf16x2(acc[qb][db][4 * g] * inv, acc[qb][db][4 * g + 1] * inv),
                           pack_bf16x2(acc[qb][db][4 * g + 2] * inv, acc[qb][db][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + dim) = w;
        }
      if (hl == 0) lse[(int64_t)bh * N + qi] = m_run[qb] * scale + logf(l_tot);
    }
  }
}

template <int D, int QB, bool CAUSAL>
hipError_t launch(const Problem& p, hipStream_t stream) {
  constexpr int BR = 32 * QB * kWaves;
  const int n_qtiles = (p.N + BR - 1) / BR;
  const int BH = p.B * p.H;
  const dim3 grid((unsigned)((int64_t)n_qtiles * BH)), block(kThreads);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, CAUSAL>), grid, block, Lds<D>::total, stream,
                     static_cast<const unsigned short*>(p.q), static_cast<const unsigned short*>(p.k),
                     static_cast<const unsigned short*>(p.v), static_cast<unsigned short*>(p.o),
                     p.lse, p.N, BH, n_qtiles, p.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const Problem& p, hipStream_t stream) {
  if (p.d == 64)
    return p.causal ? launch<64, 1, true>(p, stream) : launch<64, 1, false>(p, stream);
  return p.causal ? launch<128, 1, true>(p, stream) : launch<128, 1, false>(p, stream);
}

}  // namespace fa
