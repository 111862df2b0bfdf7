// float32 attention forward on the vector ALUs (no matrix cores).
//
// The cf-1.com FlashAttention write-up (section 4.2 and the pitfalls list of
// section 5.3) recommends getting a plain FMA version right before moving to
// matrix instructions; this kernel is that version and serves the float32
// workload.  It follows the same loop as the bf16 path: one workgroup owns a
// tile of query rows and streams K/V tiles through LDS, merging each tile
// into a running row max m, row sum l and an unnormalised accumulator with
// the rescale factor exp(m_old - m_new) (aiqz.cc Flash Attention IO article,
// section 在线Softmax算法), dividing by l once at the end.
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
  // +1 word of padding per row keeps the 8 key rows a thread group reads in
  // distinct LDS banks.
  __shared__ float Qs[kRows][D + 1];
  __shared__ float Ks[kKeys][D + 1];
  __shared__ float Vs[kKeys][D];
  __shared__ float Ps[kRows][kKeys + 1];

  const int tid = threadIdx.x;
  const int row = tid / kParts;          // query row inside the tile
  const int part = tid % kParts;         // which slice of keys / dims
  const int qt = blockIdx.x % n_qtiles;
  const int64_t bh = blockIdx.x / n_qtiles;
  const int q0 = qt * kRows;
  const int64_t head = bh * (int64_t)N * D;
  const float c = scale * 1.4426950408889634f;   // scale * log2(e)

  for (int e = tid; e < kRows * D; e += kThreads) {
    const int r = e / D, col = e % D;
    Qs[r][col] = (q0 + r < N) ? q[head + (int64_t)(q0 + r) * D + col] : 0.f;
  }

  constexpr int DP = D / kParts;          // output dims owned by a thread
  float acc[DP];
#pragma unroll
  for (int t = 0; t < DP; ++t) acc[t] = 0.f;
  float m = -INFINITY;   // running max of the raw dot products of this row
  float l = 0.f;         // this thread's share of the running sum

  const int qi = q0 + row;
  const int kv_end = causal ? min(N, q0 + kRows) : N;
  for (int k0 = 0; k0 < kv_end; k0 += kKeys) {
    __syncthreads();   // previous tile fully consumed
    for (int e = tid; e < kKeys * D; e += kThreads) {
      const int r = e / D, col = e % D;
      const bool ok = k0 + r < N;
      const int64_t g = head + (int64_t)(k0 + r) * D + col;
      Ks[r][col] = ok ? k[g] : 0.f;
      Vs[r][col] = ok ? v[g] : 0.f;
    }
    __syncthreads();

    // scores for keys part, part+8, part+16, part+24
    float s[kKeys / kParts];
    float tmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < kKeys / kParts; ++t) {
      const int kj = part + kParts * t;
      float dot = 0.f;
#pragma unroll 16
      for (int col = 0; col < D; ++col) dot = fmaf(Qs[row][col], Ks[kj][col], dot);
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
    for (int kj = 0; kj < kKeys; ++kj) {
      const float p = Ps[row][kj];
#pragma unroll
      for (int t = 0; t < DP; ++t) acc[t] = fmaf(p, Vs[kj][part * DP + t], acc[t]);
    }
  }

#pragma unroll
  for (int off = 1; off < kParts; off <<= 1) l += __shfl_xor(l, off);
  if (qi < N) {
    const float inv = 1.f / l;
    float* orow = o + head + (int64_t)qi * D + part * DP;
#pragma unroll
    for (int t = 0; t < DP; ++t) orow[t] = acc[t] * inv;
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
