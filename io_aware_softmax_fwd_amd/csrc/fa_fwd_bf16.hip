// bf16 attention forward on the gfx950 matrix cores.
//
// One workgroup owns 128 query rows of one (batch, head) and streams the K/V
// tiles of that head through LDS; the scores and probabilities of a tile live
// only in registers and are merged into a running row max m, row sum l and an
// unnormalised fp32 accumulator, which is rescaled by exp(m_old - m_new) when
// the max moves and divided by l once at the end (aiqz.cc Flash Attention IO
// article, sections 分块Tiling策略 and 在线Softmax算法; cf-1.com FlashAttention
// write-up, sections 3.2 and 4.3).  Queries are the outer loop and keys the
// inner one, so a query tile reads Q once and writes O once.
//
// Work inside a workgroup (4 waves of 64 lanes, 32 query rows per wave):
//   * scores are produced transposed, S^T = K Q^T, by
//     v_mfma_f32_32x32x16_bf16 with K (from LDS) as the A operand and Q
//     (registers, loaded once) as the B operand.  In the accumulator layout
//     lane l holds query l%32 and 16 keys of each 32-key block, so the row
//     max and row sum are in-lane reductions plus one v_permlane32_swap;
//   * the output is accumulated transposed as well, O^T += V^T P^T: the
//     probabilities are used in place as the B operand (rounded to bf16) and
//     V^T is read from row-major V in LDS with ds_read_b64_tr_b16, whose
//     16-lane transpose hands each lane 4 keys of one head dimension; two
//     such reads give the 8 keys, in the accumulator's key order, that the
//     lane's probabilities cover.
// Pipeline: K and V tiles stream straight from memory into LDS
// (buffer_load_dwordx4 ... lds, range-checked so keys past N read as zero),
// one tile ahead, double-buffered in four separate LDS arrays picked at
// compile time (the tile loop is unrolled by two); one barrier per tile.
// Separate arrays let the compiler see that the in-flight loads never touch
// the buffers being read, so the loads get the whole step to land.
// LDS rows are padded so that fragment reads hit distinct banks with every
// lane's addresses a compile-time offset from one base.
// Rescaling is lazy: the running max used as the exponent's offset only moves
// when a row's max exceeds it by more than 8/c (c = scale*log2 e), so
// probabilities stay <= 2^8 and the accumulator is rescaled rarely; since O
// and l share the offset the result is unchanged (the softmax identity holds
// for any offset; zzszmyf.github.io notes, section 5.1).
// Causal: key tiles wholly above the diagonal are never loaded, masking is
// applied only on diagonal tiles and on the ragged last tile.
#include <math.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeys = 64;                 // keys per K/V tile (Bc)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;             // log2 headroom before a rescale

template <int D> struct Cfg {
  // K rows carry one 16-byte pad chunk, so the 16-byte fragment reads of 16
  // consecutive rows fall in distinct bank groups.  V rows are padded so that
  // the four rows a transposed read touches land in four distinct quarters
  // of the banks.
  static constexpr int kStride = 2 * D + 16;           // bytes per K row
  static constexpr int vStride = D == 128 ? 320 : 192; // bytes per V row
  static constexpr int kTile = kKeys * kStride;        // bytes of one K tile
  static constexpr int vTile = kKeys * vStride;        // bytes of one V tile
  static constexpr int lds = 2 * (kTile + vTile);      // two K and two V buffers
  static constexpr int kDma = kTile / 1024;            // 1 KB LDS-DMA loads per tile
  static constexpr int vDma = vTile / 1024;
  static constexpr int kDmaPerWave = (kDma + kWaves - 1) / kWaves;
  static constexpr int vDmaPerWave = (vDma + kWaves - 1) / kWaves;
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> one word of two bf16 (round to nearest even), one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// max over both halves of the wave: lane l and lane l^32 end with the same value.
__device__ __forceinline__ float max_across_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Buffer descriptor over keys [k0, N) of one head's K or V: loads at or past
// key N are out of range and return zero.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const unsigned short* head, int k0, int N) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)(head + (int64_t)k0 * D), (short)0,
                                           (N - k0) * (2 * D), 0x00020000);
}

// Source byte offset (inside one tile of K or V) fetched by LDS-DMA slot
// `slot` of a tile whose LDS rows are `stride` bytes long; a slot in a pad
// position re-fetches the row's last chunk (never read back).
template <int D>
__device__ __forceinline__ int dma_offset(int slot, int stride) {
  const int slots = stride / 16;
  const int r = slot / slots;
  const int cc = min(slot % slots, D / 8 - 1);
  return r * (2 * D) + 16 * cc;
}

template <int D, int QB, bool CAUSAL>
struct Fwd {
  static constexpr int KS = D / 16, DB = D / 32, KB = kKeys / 32, PS = kKeys / 16;
  static constexpr int WR = 32 * QB;        // query rows per wave

  const unsigned short* kh;
  const unsigned short* vh;
  int N, wave, l32, hl, qw;
  float c, thr;
  bf16x8 qf[QB][KS];      // Q fragments (B operand of S^T = K Q^T), per 32-row block
  f32x16 acc[QB][DB];     // O^T accumulators: lane holds query l%32 of each block
  float m[QB];            // exponent offsets (raw-score units)
  float l[QB];            // this lane's share of the row sums, relative to m
  int koff[Cfg<D>::kDmaPerWave];   // source byte offsets of the K LDS-DMA slots
  int voff[Cfg<D>::vDmaPerWave];   // source byte offsets of the V LDS-DMA slots
  int k_rd, v_rd;                  // this lane's fragment read offsets in a buffer
  // LDS: K and V of two tiles, as four separate arrays selected at compile
  // time, so the compiler sees that the LDS-DMA writes into one buffer do not
  // touch the buffers being read and inserts no wait for them.
  unsigned char* kbuf[2];
  unsigned char* vbuf[2];

  __device__ int qi(int qb) const { return qw + 32 * qb + l32; }

  __device__ void setup_offsets(int lane) {
#pragma unroll
    for (int i = 0; i < Cfg<D>::kDmaPerWave; ++i)
      koff[i] = dma_offset<D>((wave + kWaves * i) * 64 + lane, Cfg<D>::kStride);
#pragma unroll
    for (int i = 0; i < Cfg<D>::vDmaPerWave; ++i)
      voff[i] = dma_offset<D>((wave + kWaves * i) * 64 + lane, Cfg<D>::vStride);
    k_rd = l32 * Cfg<D>::kStride + 16 * hl;
    // Transposed V reads: in each 16-lane group g, lane 4e + j addresses key
    // row 4*(g/2) + e and head dims 16*(g%2) + 4j .. +3 of a 32-dim block.
    const int g = lane >> 4, e = (lane >> 2) & 3, j = lane & 3;
    v_rd = (4 * (g >> 1) + e) * Cfg<D>::vStride + 2 * (16 * (g & 1) + 4 * j);
  }

  // Queue this wave's share of K (or V) of the tile at key k0 into LDS
  // buffer B (asynchronous; completion is awaited with vmcnt).
  template <bool IS_V, int B>
  __device__ void issue(int k0) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int nblk = IS_V ? Cfg<D>::vDma : Cfg<D>::kDma;
    constexpr int per_wave = IS_V ? Cfg<D>::vDmaPerWave : Cfg<D>::kDmaPerWave;
    const __amdgpu_buffer_rsrc_t r = tile_rsrc<D>(IS_V ? vh : kh, k0, N);
    unsigned char* dst = IS_V ? vbuf[B] : kbuf[B];
#pragma unroll
    for (int i = 0; i < per_wave; ++i) {
      const int blk = wave + kWaves * i;
      if (nblk % kWaves == 0 || blk < nblk)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + blk * 1024), 16,
                                                 IS_V ? voff[i] : koff[i], 0, 0, 0);
    }
#endif
  }

  // Online-softmax step of one 32-row block for the tile at key k0: moves
  // the offset when needed (rescaling its accumulator), writes the bf16
  // probabilities and adds their row sum.
  template <bool MASK>
  __device__ void softmax(int qb, f32x16 (&s)[KB], bf16x8 (&pf)[PS], int k0) {
    if constexpr (MASK) {
      // key = k0 + 32*kb + (r&3) + 8*(r>>2) + 4*hl must be <= min(qi, N-1)
      const int lim = (CAUSAL ? min(qi(qb), N - 1) : N - 1) - k0 - 4 * hl;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + (r & 3) + 8 * (r >> 2) > lim) s[kb][r] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = (kb == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = max_across_halves(mx);
    // Move the offset only when this row's max ran more than `thr` past it
    // (always on the first tile, where m = -inf).
    const bool upd = mx > m[qb] + thr;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      asm volatile("" ::: "memory");   // keep this a taken/skipped branch
      const float m_new = upd ? mx : m[qb];
      const float alpha = __builtin_amdgcn_exp2f((m[qb] - m_new) * c);   // 1 if kept, 0 at start
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
      l[qb] *= alpha;
      m[qb] = m_new;
    }
    const float mc = m[qb] * c;
    // Probabilities, rounded to bf16 for the product; the row sum is taken
    // over the same rounded values (two per v_dot2_f32_bf16), so numerator
    // and denominator see identical weights.
    float ps0 = 0.f, ps1 = 0.f;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * half + e], c, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * half + e + 1], c, -mc));
          // dot2 of the converted pair itself: taking it from an element of
          // the vector under construction is miscompiled (the same element
          // is summed repeatedly).
          const bf16x2 pb = __builtin_convertvector((f32x2{p0, p1}), bf16x2);
          if (e & 2) ps1 = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, ps1, false);
          else       ps0 = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, ps0, false);
          w[e / 2] = __builtin_bit_cast(unsigned, pb);
        }
        pf[2 * kb + half] = __builtin_bit_cast(bf16x8, w);
      }
    l[qb] += ps0 + ps1;
  }

  // Consume the tile in buffers PAR: S^T = K Q^T for every block (each K
  // fragment feeds all blocks), the softmax merges, then O^T += V^T P^T
  // (each V fragment feeds all blocks).
  template <bool MASK, int PAR>
  __device__ void consume(int k0) {
    const unsigned char* kt = kbuf[PAR] + k_rd;
    const unsigned char* vt = vbuf[PAR] + v_rd;
    f32x16 s[QB][KB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt + 32 * kb * Cfg<D>::kStride + 32 * ks);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ks], s[qb][kb], 0, 0, 0);
      }

    bf16x8 pf[QB][PS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) softmax<MASK>(qb, s[qb], pf[qb], k0);

#pragma unroll
    for (int ps = 0; ps < PS; ++ps)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const unsigned char* src = vt + 16 * ps * Cfg<D>::vStride + 64 * db;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + 8 * Cfg<D>::vStride));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][ps], acc[qb][db], 0, 0, 0);
      }
  }

  // One pipeline step: queue tile j+1 into the other buffers (it gets the
  // whole step to land), consume tile j, wait and synchronise.
  // PAR = j & 1 selects the buffers at compile time.
  template <bool MASK, int PAR>
  __device__ void step(int j, int n_tiles) {
    const int k0 = j * kKeys;
    if (j + 1 < n_tiles) {
      issue<false, PAR ^ 1>(k0 + kKeys);
      issue<true, PAR ^ 1>(k0 + kKeys);
    }
    // Causal: a wave whose last query precedes the tile's first key has
    // nothing to do here or later; the barrier below stays unconditional.
    if (!MASK || !CAUSAL || k0 <= qw + WR - 1) consume<MASK, PAR>(k0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
  }
};

template <int D, int QB, bool CAUSAL>
__global__ __launch_bounds__(kThreads, QB == 1 ? 2 : 1) void fwd_bf16_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
    const unsigned short* __restrict__ v, unsigned short* __restrict__ o,
    float* __restrict__ lse, int N, int BH, int n_qtiles, float scale) {
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds0[Cfg<D>::kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds1[Cfg<D>::kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds0[Cfg<D>::vTile];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds1[Cfg<D>::vTile];
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int BR = 32 * QB * kWaves;   // query rows per workgroup
  using F = Fwd<D, QB, CAUSAL>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Heaviest query tiles first (causal work grows with the tile index); heads
  // vary fastest, so with B*H a multiple of 8 every tile of a head lands on
  // the same XCD and shares its L2.
  const int bh = blockIdx.x % BH;
  const int qt = n_qtiles - 1 - (int)(blockIdx.x / BH);
  const int q0 = qt * BR;
  const int64_t head = (int64_t)bh * N * D;

  F f;
  f.kbuf[0] = k_lds0;
  f.kbuf[1] = k_lds1;
  f.vbuf[0] = v_lds0;
  f.vbuf[1] = v_lds1;
  f.kh = k + head;
  f.vh = v + head;
  f.N = N;
  f.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  f.l32 = lane & 31;
  f.hl = lane >> 5;
  f.qw = q0 + f.wave * F::WR;
  f.c = scale * kLog2e;
  f.thr = kLazy / f.c;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    f.m[qb] = -INFINITY;
    f.l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) f.acc[qb][db][r] = 0.f;
    const int qi = f.qi(qb);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qi < N) raw = *reinterpret_cast<const u32x4*>(q + head + (int64_t)qi * D + 16 * ks + 8 * f.hl);
      f.qf[qb][ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  f.setup_offsets(lane);

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int n_tiles = (kv_end + kKeys - 1) / kKeys;
  // Tiles before n_full need no mask: every key is < N and, when causal,
  // precedes the workgroup's first query.
  const int n_full = CAUSAL ? min(q0, N / kKeys * kKeys) / kKeys : N / kKeys;

  f.template issue<false, 0>(0);
  f.template issue<true, 0>(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int j = 0;
  for (; j + 1 < n_full; j += 2) {
    f.template step<false, 0>(j, n_tiles);
    f.template step<false, 1>(j + 1, n_tiles);
  }
  if (j < n_full) f.template step<false, 0>(j++, n_tiles);
  for (; j < n_tiles; ++j) {
    if (j & 1) f.template step<true, 1>(j, n_tiles);
    else       f.template step<true, 0>(j, n_tiles);
  }

  // Epilogue: O = acc / l in bf16 (round to nearest even), LSE = scale*m + ln l.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = sum_across_halves(f.l[qb]);
    const int qi = f.qi(qb);
    if (qi < N) {
      const float inv = 1.f / l_tot;
      unsigned short* orow = o + head + (int64_t)qi * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dim = 32 * db + 8 * g + 4 * f.hl;
          const u32x2 w = {pack_bf16x2(f.acc[qb][db][4 * g] * inv, f.acc[qb][db][4 * g + 1] * inv),
                           pack_bf16x2(f.acc[qb][db][4 * g + 2] * inv, f.acc[qb][db][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + dim) = w;
        }
      if (f.hl == 0) lse[(int64_t)bh * N + qi] = f.m[qb] * scale + logf(l_tot);
    }
  }
}

template <int D, int QB, bool CAUSAL>
hipError_t launch(const Problem& p, hipStream_t stream) {
  constexpr int BR = 32 * QB * kWaves;
  const int n_qtiles = (p.N + BR - 1) / BR;
  const int BH = p.B * p.H;
  const dim3 grid((unsigned)((int64_t)n_qtiles * BH)), block(kThreads);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, CAUSAL>), grid, block, 0, stream,
                     static_cast<const unsigned short*>(p.q), static_cast<const unsigned short*>(p.k),
                     static_cast<const unsigned short*>(p.v), static_cast<unsigned short*>(p.o),
                     p.lse, p.N, BH, n_qtiles, p.scale);
  return hipGetLastError();
}

}  // namespace

#ifndef FA_QB128
#define FA_QB128 1
#endif
#ifndef FA_QB64
#define FA_QB64 1
#endif

hipError_t launch_fwd_bf16(const Problem& p, hipStream_t stream) {
  if (p.d == 64)
    return p.causal ? launch<64, FA_QB64, true>(p, stream) : launch<64, FA_QB64, false>(p, stream);
  return p.causal ? launch<128, FA_QB128, true>(p, stream) : launch<128, FA_QB128, false>(p, stream);
}

}  // namespace fa
