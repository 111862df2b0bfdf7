// float32 attention forward on the vector ALUs (no matrix cores).
//
// The cf-1.com FlashAttention write-up (section 4.2 and the pitfalls list of
// section 5.3) recommends getting a plain FMA version right before moving to
// matrix instructions; this kernel is that version and serves the float32
// workload.  It follows the same loop as the bf16 path: one workgroup owns a
// tile of query rows and streams K/V tiles through LDS, merging each tile
// into a running row max m, row sum l and an unnormalised accumulator with
// the rescale factor exp(m_old - m_new) (aiqz.cc Flash Attention IO article,
// section 在线Softmax算法), dividing by l once at the end.  Each thread keeps
// its row's query in registers and reads K rows from LDS 16 bytes at a time;
// the next K/V tile is loaded into registers while the current one is used.
#include <math.h>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kRows = 32;        // query rows per workgroup
constexpr int kKeys = 32;        // keys per K/V tile
constexpr int kThreads = 256;    // 8 threads per query row
constexpr int kParts = kThreads / kRows;

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, float* __restrict__ o,
    float* __restrict__ lse, int N, int n_qtiles, float scale, int causal) {
  // K rows padded by 4 words: the 16-byte reads of the 8 key rows that the 8
  // threads of a row group take at once start on distinct bank quads.
  constexpr int KP = D + 4;
  __shared__ __attribute__((aligned(16))) float Ks[kKeys][KP];
  __shared__ __attribute__((aligned(16))) float Vs[kKeys][D];
  __shared__ float Ps[kRows][kKeys + 1];

  const int tid = threadIdx.x;
  const int row = tid / kParts;          // query row inside the tile
  const int part = tid % kParts;         // which slice of keys / dims
  const int qt = blockIdx.x % n_qtiles;
  const int64_t bh = blockIdx.x / n_qtiles;
  const int q0 = qt * kRows;
  const int64_t head = bh * (int64_t)N * D;
  const float c = scale * 1.4426950408889634f;   // scale * log2(e)
  const int qi = q0 + row;

  // the row's query in registers (every thread of the row group holds it)
  float4 qr[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) {
    qr[i] = float4{0.f, 0.f, 0.f, 0.f};
    if (qi < N) qr[i] = reinterpret_cast<const float4*>(q + head + (int64_t)qi * D)[i];
  }

  constexpr int DP = D / kParts;          // output dims owned by a thread
  float acc[DP];
#pragma unroll
  for (int t = 0; t < DP; ++t) acc[t] = 0.f;
  float m = -INFINITY;   // running max of the raw dot products of this row
  float l = 0.f;         // this thread's share of the running sum

  const int kv_end = causal ? min(N, q0 + kRows) : N;
  // The next tile's K and V are loaded into registers while the current
  // tile is consumed, then stored to LDS (16 bytes per thread and load).
  constexpr int PF = kKeys * D / 4 / kThreads;
  float4 kpre[PF], vpre[PF];
  auto prefetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int e = tid + i * kThreads;
      const int r = e / (D / 4), c4 = e % (D / 4);
      const int64_t g = head + (int64_t)(k0 + r) * D;
      kpre[i] = float4{0.f, 0.f, 0.f, 0.f};
      vpre[i] = float4{0.f, 0.f, 0.f, 0.f};
      if (k0 + r < N) {
        kpre[i] = reinterpret_cast<const float4*>(k + g)[c4];
        vpre[i] = reinterpret_cast<const float4*>(v + g)[c4];
      }
    }
  };
  prefetch(0);
  for (int k0 = 0; k0 < kv_end; k0 += kKeys) {
    __syncthreads();   // previous tile fully consumed
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int e = tid + i * kThreads;
      const int r = e / (D / 4), c4 = e % (D / 4);
      *reinterpret_cast<float4*>(&Ks[r][4 * c4]) = kpre[i];
      *reinterpret_cast<float4*>(&Vs[r][4 * c4]) = vpre[i];
    }
    __syncthreads();
    if (k0 + kKeys < kv_end) prefetch(k0 + kKeys);

    // scores for keys part, part+8, part+16, part+24
    float s[kKeys / kParts];
    float tmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < kKeys / kParts; ++t) {
      const int kj = part + kParts * t;
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) {
        const float4 kk = *reinterpret_cast<const float4*>(&Ks[kj][4 * i]);
        dot = fmaf(qr[i].x, kk.x, dot);
        dot = fmaf(qr[i].y, kk.y, dot);
        dot = fmaf(qr[i].z, kk.z, dot);
        dot = fmaf(qr[i].w, kk.w, dot);
      }
      const int key = k0 + kj;
      const bool masked = key >= N || (causal && key > qi);
      s[t] = masked ? -INFINITY : dot;
      tmax = fmaxf(tmax, s[t]);
    }
    // row max across the 8 threads of the row (adjacent lanes of one wave)
#pragma unroll
    for (int off = 1; off < kParts; off <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));
    const float m_new = fmaxf(m, tmax);
    const float mc = m_new * c;
    const float r = exp2f(m * c - mc);      // 0 on the first tile (m = -inf)
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < kKeys / kParts; ++t) {
      const float p = exp2f(fmaf(s[t], c, -mc));
      psum += p;
      Ps[row][part + kParts * t] = p;
    }
    l = l * r + psum;
    m = m_new;
    __syncthreads();   // P visible to the whole row group
#pragma unroll
    for (int t = 0; t < DP; ++t) acc[t] *= r;
#pragma unroll 4
    for (int kj = 0; kj < kKeys; ++kj) {
      const float p = Ps[row][kj];
#pragma unroll
      for (int t = 0; t < DP; t += 4) {
        const float4 vv = *reinterpret_cast<const float4*>(&Vs[kj][part * DP + t]);
        acc[t] = fmaf(p, vv.x, acc[t]);
        acc[t + 1] = fmaf(p, vv.y, acc[t + 1]);
        acc[t + 2] = fmaf(p, vv.z, acc[t + 2]);
        acc[t + 3] = fmaf(p, vv.w, acc[t + 3]);
      }
    }
  }

#pragma unroll
  for (int off = 1; off < kParts; off <<= 1) l += __shfl_xor(l, off);
  if (qi < N) {
    const float inv = 1.f / l;
    float* orow = o + head + (int64_t)qi * D + part * DP;
#pragma unroll
    for (int t = 0; t < DP; t += 4)
      *reinterpret_cast<float4*>(orow + t) = float4{acc[t] * inv, acc[t + 1] * inv, acc[t + 2] * inv, acc[t + 3] * inv};
    if (part == 0) lse[bh * (int64_t)N + qi] = m * scale + logf(l);
  }
}

}  // namespace

hipError_t launch_fwd_f32(const Problem& p, hipStream_t stream) {
  const int n_qtiles = (p.N + kRows - 1) / kRows;
  const int64_t blocks = (int64_t)n_qtiles * p.B * p.H;
  const dim3 grid((unsigned)blocks), block(kThreads);
  const float* q = static_cast<const float*>(p.q);
  const float* k = static_cast<const float*>(p.k);
  const float* v = static_cast<const float*>(p.v);
  float* o = static_cast<float*>(p.o);
  if (p.d == 64)
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, stream, q, k, v, o,
                       p.lse, p.N, n_qtiles, p.scale, p.causal);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, stream, q, k, v, o,
                       p.lse, p.N, n_qtiles, p.scale, p.causal);
  return hipGetLastError();
}

}  // namespace fa
