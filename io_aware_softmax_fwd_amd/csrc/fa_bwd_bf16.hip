// bf16 attention backward on the gfx950 matrix cores, by recomputation.
//
// The forward pass keeps only O and one log-sum-exp per row; the backward
// pass re-reads Q, K, V in tiles and rebuilds the scores and probabilities
// on chip instead of storing the N x N matrices (zzszmyf.github.io notes
// "FlashAttention 原理是什么", section 6; aiqz.cc Flash Attention IO article,
// section 工程实现细节).  With P = exp(scale*QK^T - LSE) (row statistics
// from the forward pass) the gradients are the chain rule
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D_i = <dO_i, O_i>,
//     dQ = scale * dS K,   dK = scale * dS^T Q
// (D_i equals sum_j P_ij dP_ij because O_i = sum_j P_ij v_j).
//
// Two kernels, no atomics, so every result is reproducible bit for bit:
//   bwd_dq_kernel    one workgroup per 128 query rows.  Q and dO stay in
//                    registers, K and V tiles stream through LDS; it also
//                    writes D for the second kernel.  Products are taken
//                    transposed as in the forward kernel (S^T = K Q^T,
//                    dP^T = V dO^T, dQ^T += K^T dS^T) so each lane owns one
//                    query and its row statistics are lane constants.
//   bwd_dkdv_kernel  one workgroup per 128 keys.  K and V stay in registers,
//                    Q and dO tiles (with the rows' LSE and D) stream through
//                    LDS; S = Q K^T and dP = dO V^T put one key per lane, and
//                    dV^T += dO^T P, dK^T += Q^T dS take the probabilities
//                    straight from the accumulators as B operands, with the
//                    transposed operand read by ds_read_b64_tr_b16.
// Both recompute S and dP: seven N^2 d products in all against five for a
// single kernel that adds dQ with atomics, traded for determinism.  When
// neither grid alone would fill the GPU (at most 128 workgroups each), D is
// written by a small row-dot kernel first and the two kernels' workgroups
// run as one launch (bwd_fused_kernel), side by side.
#include <math.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kRows = 64;        // rows per streamed tile (keys, or queries)

// LDS row strides in bytes.  An operand read only row-major (16-byte
// fragment reads, 16 consecutive rows per access group) uses 2D + 16
// bytes: stride/4 is 4 (mod 64) banks times an odd number, so the 16 rows
// start on distinct bank quads.  An operand read both row-major and
// transposed (ds_read_b64_tr_b16: 4 rows x 32 bytes per 32 lanes) uses
// stride/4 = 12 (d=128) or 52 (d=64) mod 64: still conflict-free row
// reads, and at most 2-way conflicts on the transposed reads.
template <int D> struct BwdCfg {
  static constexpr int rowStride = 2 * D + 16;
  static constexpr int bothStride = D == 128 ? 304 : 208;
};

// LDS-DMA of one 64-row tile of a [N, D] bf16 head into an LDS buffer of
// STRIDE-byte rows, spread over the four waves in 1 KB blocks.
template <int D, int STRIDE> struct Dma {
  static constexpr int bytes = kRows * STRIDE;
  static constexpr int nblk = bytes / 1024;
  static constexpr int perWave = (nblk + kBwdWaves - 1) / kBwdWaves;
  static_assert(bytes % 1024 == 0, "tile must be whole 1 KB blocks");
  int off[perWave];
  __device__ void setup(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < perWave; ++i) off[i] = dma_offset<D>((wave + kBwdWaves * i) * 64 + lane, STRIDE);
  }
  __device__ void issue(const unsigned short* head, int r0, int N, unsigned char* dst, int wave) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t r = tile_rsrc<D>(head, r0, N);
#pragma unroll
    for (int i = 0; i < perWave; ++i) {
      const int blk = wave + kBwdWaves * i;
      if (nblk % kBwdWaves == 0 || blk < nblk)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + blk * 1024), 16, off[i], 0, 0, 0);
    }
#endif
  }
};

// Transposed 32-row x 16-key operand from a row-major LDS tile: `src` is this
// lane's address of key row 0 of the 16-key group; the two reads (rows +0 and
// +8) give the 8 keys that the accumulator layout assigns to the lane.
template <int STRIDE>
__device__ __forceinline__ bf16x8 tr_operand(const unsigned char* src) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + 8 * STRIDE));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Lane offset of the transposed reads: in each 16-lane group g, lane 4e + j
// addresses row 4*(g/2) + e and columns 16*(g%2) + 4j .. +3 of a 32-column
// block.
template <int STRIDE>
__device__ __forceinline__ int tr_offset(int lane) {
  const int g = lane >> 4, e = (lane >> 2) & 3, j = lane & 3;
  return (4 * (g >> 1) + e) * STRIDE + 2 * (16 * (g & 1) + 4 * j);
}

// Load this lane's share of one row as MFMA B-operand fragments: dims
// 16*ks + 8*hl .. +7 for ks < D/16 (zero when the row is out of range).
template <int D>
__device__ __forceinline__ void load_row_fragments(const unsigned short* row, bool valid, int hl,
                                                   bf16x8 (&f)[D / 16]) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (valid) raw = *reinterpret_cast<const u32x4*>(row + 16 * ks + 8 * hl);
    f[ks] = __builtin_bit_cast(bf16x8, raw);
  }
}

// Store a transposed fp32 accumulator (rows = head dims, lane = one output
// row) times `mul` as bf16: dims 32*db + 8*g + 4*hl .. +3 from elements
// 4g .. 4g+3 of block db.
template <int D>
__device__ __forceinline__ void store_rowT(unsigned short* row, const f32x16 (&acc)[D / 32], float mul,
                                           int hl) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dim = 32 * db + 8 * g + 4 * hl;
      const u32x2 w = {pack_bf16x2(acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul),
                       pack_bf16x2(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul)};
      *reinterpret_cast<u32x2*>(row + dim) = w;
    }
}

// The same rows as fp32 (partial sums of a group of query heads).
template <int D>
__device__ __forceinline__ void store_rowT_f32(float* row, const f32x16 (&acc)[D / 32], float mul, int hl) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dim = 32 * db + 8 * g + 4 * hl;
      const float4 w = {acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul, acc[db][4 * g + 2] * mul,
                        acc[db][4 * g + 3] * mul};
      *reinterpret_cast<float4*>(row + dim) = w;
    }
}

// K/V head read by query head bh (of B*H) when G query heads share one.
__device__ __forceinline__ int kv_head(int bh, int H, int G) { return (bh / H) * (H / G) + (bh % H) / G; }

// ----------------------------------------------------------------- dQ kernel
template <int D, bool CAUSAL>
struct BwdQ {
  static constexpr int KS = D / 16, DB = D / 32;
  static constexpr int KSTR = BwdCfg<D>::bothStride, VSTR = BwdCfg<D>::rowStride;

  const unsigned short* kh;
  const unsigned short* vh;
  int N, wave, l32, hl, qi;
  float c, lse2, Drow;
  bf16x8 qf[KS];          // Q row of this lane's query (B operand of S^T = K Q^T)
  bf16x8 gf[KS];          // dO row (B operand of dP^T = V dO^T)
  f32x16 acc[DB];         // dQ^T: lane holds query l%32
  Dma<D, KSTR> kd;
  Dma<D, VSTR> vd;
  int k_rd, v_rd, kt_rd;
  unsigned char* kbuf[2];
  unsigned char* vbuf[2];

  template <int B>
  __device__ void issue(int k0) {
    kd.issue(kh, k0, N, kbuf[B], wave);
    vd.issue(vh, k0, N, vbuf[B], wave);
  }

  template <bool MASK, int PAR>
  __device__ void consume(int k0) {
    const unsigned char* kt = kbuf[PAR];
    const unsigned char* vt = vbuf[PAR];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt + k_rd + 32 * h2 * KSTR + 32 * ks);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vt + v_rd + 32 * h2 * VSTR + 32 * ks);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, gf[ks], dp, 0, 0, 0);
      }
      // dS^T = P^T (dP^T - D); key = k0 + 32*h2 + (r&3) + 8*(r>>2) + 4*hl
      const int lim = (CAUSAL ? min(qi, N - 1) : N - 1) - k0 - 32 * h2 - 4 * hl;
      bf16x8 dsf[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int r = 8 * half + e;
          float p0 = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lse2));
          float p1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], c, -lse2));
          if (MASK) {
            if ((r & 3) + 8 * (r >> 2) > lim) p0 = 0.f;
            if (((r + 1) & 3) + 8 * ((r + 1) >> 2) > lim) p1 = 0.f;
          }
          w[e / 2] = pack_bf16x2(p0 * (dp[r] - Drow), p1 * (dp[r + 1] - Drow));
        }
        dsf[half] = __builtin_bit_cast(bf16x8, w);
      }
      // dQ^T += K^T dS^T over the 32 keys, two 16-key steps
#pragma unroll
      for (int ps = 0; ps < 2; ++ps)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 kT = tr_operand<KSTR>(kt + kt_rd + (32 * h2 + 16 * ps) * KSTR + 64 * db);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kT, dsf[ps], acc[db], 0, 0, 0);
        }
    }
  }

  template <bool MASK, int PAR>
  __device__ void step(int j, int t_end, int wlast) {
    const int k0 = j * kRows;
    if (j + 1 < t_end) issue<PAR ^ 1>(k0 + kRows);
    if (!MASK || !CAUSAL || k0 <= wlast) consume<MASK, PAR>(k0);
    // The waits are the builtin, not inline assembly: the compiler then knows
    // that the loads before them have landed and does not wait for them again
    // (such a wait, placed after the next tile's loads were queued, would wait
    // for those too).
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
  }
};

// D_i = <dO_i, O_i> of this lane's row: its 64 dims (half hl of the row),
// then the other half-wave's.  The dQ kernel and the row-dot kernel share
// it, so both produce the same bits.
template <int D>
__device__ __forceinline__ float row_dot(const unsigned short* orow, bool valid, int hl,
                                         const bf16x8 (&gf)[D / 16]) {
  bf16x8 of[D / 16];
  load_row_fragments<D>(orow, valid, hl, of);
  float part = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2 a = {gf[ks][e], gf[ks][e + 1]};
      const bf16x2 b = {of[ks][e], of[ks][e + 1]};
      part = __builtin_amdgcn_fdot2_f32_bf16(a, b, part, false);
    }
  return sum_across_halves(part);
}

// One dQ workgroup (block `blk` of n_qtiles * BH).  WRITE_D: also store D
// for the dK/dV kernel (the fused small-grid launch has it written first).
template <int D, bool CAUSAL, bool WRITE_D>
__device__ __forceinline__ void dq_block(
    int blk, const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
    const unsigned short* __restrict__ v, const unsigned short* __restrict__ o,
    const unsigned short* __restrict__ dout, const float* __restrict__ lse,
    unsigned short* __restrict__ dq, float* __restrict__ dws, int N, int BH, int n_qtiles,
    float scale, int hg, int H, int G) {
  using F = BwdQ<D, CAUSAL>;
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds0[Dma<D, F::KSTR>::bytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds1[Dma<D, F::KSTR>::bytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds0[Dma<D, F::VSTR>::bytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds1[Dma<D, F::VSTR>::bytes];
  constexpr int DB = D / 32, BR = 32 * kBwdWaves;

  const int tid = threadIdx.x, lane = tid & 63;
  int bh, rank;
  xcd_order(blk, BH, n_qtiles, hg, bh, rank);
  const int qt = n_qtiles - 1 - rank;   // heaviest causal tiles first
  const int q0 = qt * BR;
  const int64_t head = (int64_t)bh * N * D;
  const int64_t kvh = (int64_t)kv_head(bh, H, G) * N * D;

  F f;
  f.kbuf[0] = k_lds0;
  f.kbuf[1] = k_lds1;
  f.vbuf[0] = v_lds0;
  f.vbuf[1] = v_lds1;
  f.kh = k + kvh;
  f.vh = v + kvh;
  f.N = N;
  f.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  f.l32 = lane & 31;
  f.hl = lane >> 5;
  const int qw = q0 + 32 * f.wave;
  f.qi = qw + f.l32;
  f.c = scale * kLog2e;
  const bool valid = f.qi < N;
  const unsigned short* qrow = q + head + (int64_t)f.qi * D;
  load_row_fragments<D>(qrow, valid, f.hl, f.qf);
  load_row_fragments<D>(dout + head + (int64_t)f.qi * D, valid, f.hl, f.gf);
  f.Drow = row_dot<D>(o + head + (int64_t)f.qi * D, valid, f.hl, f.gf);
  f.lse2 = valid ? lse[(int64_t)bh * N + f.qi] * kLog2e : 0.f;
  if (WRITE_D && valid && f.hl == 0) dws[(int64_t)bh * N + f.qi] = f.Drow;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) f.acc[db][r] = 0.f;
  f.kd.setup(f.wave, lane);
  f.vd.setup(f.wave, lane);
  f.k_rd = f.l32 * F::KSTR + 16 * f.hl;
  f.v_rd = f.l32 * F::VSTR + 16 * f.hl;
  f.kt_rd = tr_offset<F::KSTR>(lane);

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int n_tiles = (kv_end + kRows - 1) / kRows;
  const int n_full = CAUSAL ? min(q0 + 1, N) / kRows : N / kRows;
  const int wlast = qw + 31;   // last query of the wave (causal skip)

  f.template issue<0>(0);
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
  __syncthreads();
  int j = 0;
  const int full_end = min(n_tiles, n_full);
  for (; j + 1 < full_end; j += 2) {
    f.template step<false, 0>(j, n_tiles, wlast);
    f.template step<false, 1>(j + 1, n_tiles, wlast);
  }
  if (j < full_end) {
    f.template step<false, 0>(j, n_tiles, wlast);
    ++j;
  }
  for (; j < n_tiles; ++j) {
    if (j & 1) f.template step<true, 1>(j, n_tiles, wlast);
    else       f.template step<true, 0>(j, n_tiles, wlast);
  }
  if (valid) store_rowT<D>(dq + head + (int64_t)f.qi * D, f.acc, scale, f.hl);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dq_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
    const unsigned short* __restrict__ v, const unsigned short* __restrict__ o,
    const unsigned short* __restrict__ dout, const float* __restrict__ lse,
    unsigned short* __restrict__ dq, float* __restrict__ dws, int N, int BH, int n_qtiles,
    float scale, int hg, int H, int G) {
  dq_block<D, CAUSAL, true>(blockIdx.x, q, k, v, o, dout, lse, dq, dws, N, BH, n_qtiles, scale, hg, H, G);
}

// ------------------------------------------------------------- dK/dV kernel
template <int D, bool CAUSAL>
struct BwdKV {
  static constexpr int KS = D / 16, DB = D / 32;
  static constexpr int STR = BwdCfg<D>::bothStride;

  const unsigned short* qh;
  const unsigned short* gh;
  const float* lseh;
  const float* dh;
  int N, wave, lane, l32, hl, kj;
  float c;
  bf16x8 kf[KS];          // K row of this lane's key (B operand of S = Q K^T)
  bf16x8 vf[KS];          // V row (B operand of dP = dO V^T)
  f32x16 dk[DB];          // dK^T: lane holds key l%32
  f32x16 dv[DB];          // dV^T
  Dma<D, STR> qd;
  Dma<D, STR> gd;
  int q_rd, t_rd;
  float stat;             // waves 0 and 1: the LSE or D of row `lane` of the next tile (0 past N)
  unsigned char* qbuf[2];
  unsigned char* gbuf[2];
  float* lbuf[2];
  float* dbuf[2];

  // Queue tile q0: LSE and D into registers of waves 0 and 1 first (range-
  // checked, so rows past N read 0, and left untouched until publish, so
  // that nothing waits for them before the step's closing wait), then Q and
  // dO by LDS-DMA.
  template <int B>
  __device__ void issue(int q0) {
#if defined(__HIP_DEVICE_COMPILE__)
    if (wave < 2) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((wave == 0 ? lseh : dh) + q0), (short)0, (N - q0) * 4, 0x00020000);
      stat = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * lane, 0, 0));
    }
#endif
    qd.issue(qh, q0, N, qbuf[B], wave);
    gd.issue(gh, q0, N, gbuf[B], wave);
  }
  // After the loads of tile q0 have landed: make its row statistics visible
  // (LSE scaled by log2(e); rows >= N get LSE = +inf, hence P = 0, and D = 0).
  template <int B>
  __device__ void publish(int q0) {
    if (wave == 0) lbuf[B][lane] = q0 + lane < N ? stat * kLog2e : INFINITY;
    else if (wave == 1) dbuf[B][lane] = stat;
  }

  template <bool MASK, int PAR>
  __device__ void consume(int q0) {
    const unsigned char* qt = qbuf[PAR];
    const unsigned char* gt = gbuf[PAR];
    const float* lt = lbuf[PAR];
    const float* dt = dbuf[PAR];
    // The two 32-query halves run as a loop, not unrolled: two copies in
    // flight need more registers than a wave has.  Halves wholly
    // above the diagonal are still computed (their probabilities are 0);
    // skipping them made the accumulators pass through a branch merge that
    // the compiler could only serve by spilling.
#pragma unroll 1
    for (int h2 = 0; h2 < 2; ++h2) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qt + q_rd + 32 * h2 * STR + 32 * ks);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s, 0, 0, 0);
        const bf16x8 ga = *reinterpret_cast<const bf16x8*>(gt + q_rd + 32 * h2 * STR + 32 * ks);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf[ks], dp, 0, 0, 0);
      }
      // row statistics of the lane's 16 queries: 32*h2 + 8t + 4*hl + (0..3)
      float4 L[4], Dd[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        L[t] = *reinterpret_cast<const float4*>(lt + 32 * h2 + 8 * t + 4 * hl);
        Dd[t] = *reinterpret_cast<const float4*>(dt + 32 * h2 + 8 * t + 4 * hl);
      }
      // query of element r: q0 + 32*h2 + (r&3) + 8*(r>>2) + 4*hl; key kj
      const int qmin = kj - (q0 + 32 * h2 + 4 * hl);   // masked when (r&3) + 8*(r>>2) < qmin
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 wp, wd;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int r = 8 * half + e;
          const float* Lr = reinterpret_cast<const float*>(&L[r >> 2]);
          const float* Dr = reinterpret_cast<const float*>(&Dd[r >> 2]);
          float s0 = s[r], s1 = s[r + 1];
          if (MASK && CAUSAL) {
            if ((r & 3) + 8 * (r >> 2) < qmin) s0 = -INFINITY;
            if (((r + 1) & 3) + 8 * ((r + 1) >> 2) < qmin) s1 = -INFINITY;
          }
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s0, c, -Lr[r & 3]));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s1, c, -Lr[(r + 1) & 3]));
          wp[e / 2] = pack_bf16x2(p0, p1);
          wd[e / 2] = pack_bf16x2(p0 * (dp[r] - Dr[r & 3]), p1 * (dp[r + 1] - Dr[(r + 1) & 3]));
        }
        pf[half] = __builtin_bit_cast(bf16x8, wp);
        dsf[half] = __builtin_bit_cast(bf16x8, wd);
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the 32 queries
#pragma unroll
      for (int ps = 0; ps < 2; ++ps)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int src = t_rd + (32 * h2 + 16 * ps) * STR + 64 * db;
          const bf16x8 gT = tr_operand<STR>(gt + src);
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gT, pf[ps], dv[db], 0, 0, 0);
          const bf16x8 qT = tr_operand<STR>(qt + src);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qT, dsf[ps], dk[db], 0, 0, 0);
        }
    }
  }

  // Consume tile j from buffers PAR while tile `next` (if any) lands in the
  // other buffers.
  template <bool MASK, int PAR>
  __device__ void step(int j, int next, bool has_next) {
    if (has_next) issue<PAR ^ 1>(next * kRows);
    consume<MASK, PAR>(j * kRows);
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    if (has_next) publish<PAR ^ 1>(next * kRows);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
  }
};

// One dK/dV workgroup (block `blk` of ceil(N/128) * BH).
template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_block(
    int blk, const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
    const unsigned short* __restrict__ v, const unsigned short* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ dws, unsigned short* __restrict__ dk,
    unsigned short* __restrict__ dv, int N, int BH, float scale, int hg, int H, int G,
    float* __restrict__ pdk, float* __restrict__ pdv) {
  using F = BwdKV<D, CAUSAL>;
  __shared__ __attribute__((aligned(1024))) unsigned char q_lds0[Dma<D, F::STR>::bytes];
  __shared__ __attribute__((aligned(1024))) unsigned char q_lds1[Dma<D, F::STR>::bytes];
  __shared__ __attribute__((aligned(1024))) unsigned char g_lds0[Dma<D, F::STR>::bytes];
  __shared__ __attribute__((aligned(1024))) unsigned char g_lds1[Dma<D, F::STR>::bytes];
  __shared__ __attribute__((aligned(16))) float l_lds0[kRows];
  __shared__ __attribute__((aligned(16))) float l_lds1[kRows];
  __shared__ __attribute__((aligned(16))) float d_lds0[kRows];
  __shared__ __attribute__((aligned(16))) float d_lds1[kRows];
  constexpr int DB = D / 32, BK = 32 * kBwdWaves;

  const int tid = threadIdx.x, lane = tid & 63;
  int bh, kt;   // smallest keys first: they meet the most causal queries
  xcd_order(blk, BH, (N + BK - 1) / BK, hg, bh, kt);
  const int k0 = kt * BK;
  const int64_t head = (int64_t)bh * N * D;
  const int64_t kvh = (int64_t)kv_head(bh, H, G) * N * D;

  F f;
  f.qbuf[0] = q_lds0;
  f.qbuf[1] = q_lds1;
  f.gbuf[0] = g_lds0;
  f.gbuf[1] = g_lds1;
  f.lbuf[0] = l_lds0;
  f.lbuf[1] = l_lds1;
  f.dbuf[0] = d_lds0;
  f.dbuf[1] = d_lds1;
  f.qh = q + head;
  f.gh = dout + head;
  f.lseh = lse + (int64_t)bh * N;
  f.dh = dws + (int64_t)bh * N;
  f.N = N;
  f.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  f.lane = lane;
  f.l32 = lane & 31;
  f.hl = lane >> 5;
  f.kj = k0 + 32 * f.wave + f.l32;
  f.c = scale * kLog2e;
  const bool valid = f.kj < N;
  load_row_fragments<D>(k + kvh + (int64_t)f.kj * D, valid, f.hl, f.kf);
  load_row_fragments<D>(v + kvh + (int64_t)f.kj * D, valid, f.hl, f.vf);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      f.dk[db][r] = 0.f;
      f.dv[db][r] = 0.f;
    }
  f.qd.setup(f.wave, lane);
  f.gd.setup(f.wave, lane);
  f.q_rd = f.l32 * F::STR + 16 * f.hl;
  f.t_rd = tr_offset<F::STR>(lane);

  // Query tiles that see any of this workgroup's keys: [t0, t1).  Causal:
  // the two tiles t0 and t0 + 1 cover the workgroup's own 128 positions and
  // hold queries that precede some of its keys, so they are masked; every
  // later tile is whole.  The masked pair goes first, from buffers 0 and 1,
  // so that the whole tiles after it start on buffer 0 as well and every
  // step's buffers are fixed at compile time (a buffer chosen at run time
  // merges two copies of the step in one loop, which the compiler serves by
  // spilling).  The whole tiles are walked down from t1 - 1, so the
  // workgroups of a head sweep the same Q and dO tiles at about the same
  // time.
  static_assert(BK == 2 * kRows, "the diagonal of a workgroup spans two query tiles");
  const int t0 = CAUSAL ? k0 / kRows : 0;
  const int t1 = (N + kRows - 1) / kRows;
  const int t_full = CAUSAL ? min(t1, t0 + 2) : t0;

  if (t0 < t1) {
    const int first = CAUSAL ? t0 : t1 - 1;
    f.template issue<0>(first * kRows);
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    f.template publish<0>(first * kRows);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __syncthreads();
    if constexpr (CAUSAL) {
      // t0, then t0 + 1 if it exists; the whole tiles follow from t1 - 1
      if (t0 + 1 < t1) {
        f.template step<true, 0>(t0, t0 + 1, true);
        f.template step<true, 1>(t0 + 1, t1 - 1, t1 - 1 >= t_full);
      } else {
        f.template step<true, 0>(t0, 0, false);
      }
    }
    int j = t1 - 1;
    for (; j - 1 >= t_full; j -= 2) {
      f.template step<false, 0>(j, j - 1, true);
      f.template step<false, 1>(j - 1, j - 2, j - 2 >= t_full);
    }
    if (j >= t_full) f.template step<false, 0>(j, 0, false);
  }
  if (valid) {
    if (G == 1) {
      store_rowT<D>(dk + head + (int64_t)f.kj * D, f.dk, scale, f.hl);
      store_rowT<D>(dv + head + (int64_t)f.kj * D, f.dv, 1.f, f.hl);
    } else {
      // this query head's share; the group's shares are summed afterwards
      store_rowT_f32<D>(pdk + head + (int64_t)f.kj * D, f.dk, scale, f.hl);
      store_rowT_f32<D>(pdv + head + (int64_t)f.kj * D, f.dv, 1.f, f.hl);
    }
  }
}

// Two workgroups per CU (2 x 77 KB of LDS at d = 128): 256 registers a
// lane.  The causal d = 128 variant keeps a few values in scratch, reloaded
// around its two masked steps (once per workgroup); the loop over the whole
// tiles stays in registers.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dkdv_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
    const unsigned short* __restrict__ v, const unsigned short* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ dws, unsigned short* __restrict__ dk,
    unsigned short* __restrict__ dv, int N, int BH, float scale, int hg, int H, int G,
    float* __restrict__ pdk, float* __restrict__ pdv) {
  dkdv_block<D, CAUSAL>(blockIdx.x, q, k, v, dout, lse, dws, dk, dv, N, BH, scale, hg, H, G, pdk, pdv);
}

// D_i = <dO_i, O_i> of every row into the workspace, for the fused launch
// below (one wave per 32 rows, lanes as in the dQ kernel).
template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_rowdot_kernel(const unsigned short* __restrict__ o,
                                                                 const unsigned short* __restrict__ dout,
                                                                 float* __restrict__ dws, int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * kBwdWaves + (threadIdx.x >> 6)) * 32 + (lane & 31);
  const bool valid = row < rows;
  const int hl = lane >> 5;
  bf16x8 gf[D / 16];
  load_row_fragments<D>(dout + row * D, valid, hl, gf);
  const float dr = row_dot<D>(o + row * D, valid, hl, gf);
  if (valid && hl == 0) dws[row] = dr;
}

// Small grids: the dQ and the dK/dV workgroups in one launch (blocks below
// n_dq take the dQ work), so that they run side by side when neither grid
// alone fills the GPU.  D comes from bwd_rowdot_kernel, launched first.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_fused_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
    const unsigned short* __restrict__ v, const unsigned short* __restrict__ o,
    const unsigned short* __restrict__ dout, const float* __restrict__ lse,
    unsigned short* __restrict__ dq, unsigned short* __restrict__ dk, unsigned short* __restrict__ dv,
    float* __restrict__ dws, int N, int BH, int n_qtiles, float scale, int hg, int H, int G,
    float* __restrict__ pdk, float* __restrict__ pdv) {
  const int n_dq = n_qtiles * BH;
  if ((int)blockIdx.x < n_dq)
    dq_block<D, CAUSAL, false>(blockIdx.x, q, k, v, o, dout, lse, dq, dws, N, BH, n_qtiles, scale, hg, H, G);
  else
    dkdv_block<D, CAUSAL>(blockIdx.x - n_dq, q, k, v, dout, lse, dws, dk, dv, N, BH, scale, hg, H, G, pdk, pdv);
}

// dK and dV of each K/V head: the sum of its G query heads' fp32 shares, in
// head order (a fixed order, so the result is reproducible), rounded to
// bf16.  One thread per (K/V head row, 8 head dims).
template <int D>
__global__ __launch_bounds__(256) void bwd_group_sum_kernel(const float* __restrict__ pdk,
                                                            const float* __restrict__ pdv,
                                                            unsigned short* __restrict__ dk,
                                                            unsigned short* __restrict__ dv,
                                                            int64_t kv_rows, int N, int G) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = t / (D / 8);            // row of [B*Hkv*N]
  const int c8 = (int)(t % (D / 8));
  if (row >= kv_rows) return;
  const int64_t bkv = row / N, n = row % N;
  const int64_t first = (bkv * G * N + n) * D + 8 * c8;   // query head bkv*G, same row
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const float* src = (which ? pdv : pdk) + first;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < G; ++g) {
      const float4 a = *reinterpret_cast<const float4*>(src + (int64_t)g * N * D);
      const float4 b = *reinterpret_cast<const float4*>(src + (int64_t)g * N * D + 4);
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
    const u32x4 out = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                       pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    *reinterpret_cast<u32x4*>((which ? dv : dk) + row * D + 8 * c8) = out;
  }
}

// Up to this many workgroups in all (the dQ and the dK/dV grids together,
// one workgroup per CU of the 256 at the fused kernel's LDS use), the two
// kernels run as one launch.
constexpr int64_t kBwdFusedMaxGrid = 256;

template <int D, bool CAUSAL>
hipError_t launch_bwd(const BwdProblem& p, hipStream_t stream) {
  const int BH = p.B * p.H;
  const int G = p.H / p.Hkv;
  const int n_qtiles = (p.N + 32 * kBwdWaves - 1) / (32 * kBwdWaves);
  const int hg = xcd_head_group(BH, n_qtiles, 1, CAUSAL ? n_qtiles : 0, 1);
  const unsigned short* q = static_cast<const unsigned short*>(p.q);
  const unsigned short* k = static_cast<const unsigned short*>(p.k);
  const unsigned short* v = static_cast<const unsigned short*>(p.v);
  const unsigned short* dout = static_cast<const unsigned short*>(p.dout);
  const unsigned short* o = static_cast<const unsigned short*>(p.o);
  float* dws = static_cast<float*>(p.workspace);
  const BwdLayout L = bwd_layout(p.B, p.H, p.Hkv, p.N, D);
  unsigned char* ws = static_cast<unsigned char*>(p.workspace);
  float* pdk = G > 1 ? reinterpret_cast<float*>(ws + L.dk_offset) : nullptr;
  float* pdv = G > 1 ? reinterpret_cast<float*>(ws + L.dv_offset) : nullptr;
  unsigned short* dq = static_cast<unsigned short*>(p.dq);
  unsigned short* dk = static_cast<unsigned short*>(p.dk);
  unsigned short* dv = static_cast<unsigned short*>(p.dv);
  const int64_t grid = (int64_t)n_qtiles * BH;   // workgroups of each of the two kernels
  hipError_t e;
  if (2 * grid <= kBwdFusedMaxGrid) {
    const int64_t rows = (int64_t)BH * p.N;
    hipLaunchKernelGGL((bwd_rowdot_kernel<D>), dim3((unsigned)((rows + 32 * kBwdWaves - 1) / (32 * kBwdWaves))),
                       dim3(kBwdThreads), 0, stream, o, dout, dws, rows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_fused_kernel<D, CAUSAL>), dim3((unsigned)(2 * grid)), dim3(kBwdThreads), 0, stream,
                       q, k, v, o, dout, p.lse, dq, dk, dv, dws, p.N, BH, n_qtiles, p.scale, hg, p.H, G, pdk, pdv);
  } else {
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kBwdThreads), 0, stream,
                       q, k, v, o, dout, p.lse, dq, dws, p.N, BH, n_qtiles, p.scale, hg, p.H, G);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kBwdThreads), 0, stream,
                       q, k, v, dout, p.lse, dws, dk, dv, p.N, BH, p.scale, hg, p.H, G, pdk, pdv);
  }
  e = hipGetLastError();
  if (e != hipSuccess || G == 1) return e;
  const int64_t kv_rows = (int64_t)p.B * p.Hkv * p.N;
  const int64_t threads = kv_rows * (D / 8);
  hipLaunchKernelGGL((bwd_group_sum_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, pdk, pdv, static_cast<unsigned short*>(p.dk), static_cast<unsigned short*>(p.dv),
                     kv_rows, p.N, G);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdProblem& p, hipStream_t stream) {
  if (p.d == 64) return p.causal ? launch_bwd<64, true>(p, stream) : launch_bwd<64, false>(p, stream);
  return p.causal ? launch_bwd<128, true>(p, stream) : launch_bwd<128, false>(p, stream);
}

}  // namespace fa
