// fp8 attention forward with per-block scales on the gfx950 matrix cores.
//
// The low-precision variant quantizes Q, K and V block by block, each block
// with its own scale (zzszmyf.github.io notes "FlashAttention 原理是什么",
// section 10 item ③ and section 12.2).  Blocks here are the 32-element
// blocks of the MX layout that v_mfma_scale_f32_32x32x64_f8f6f4 consumes:
// E4M3 codes plus one E8M0 power-of-two scale per 32 consecutive elements of
// the contracted dimension, applied by the matrix core itself.
//   Q, K : blocks of 32 consecutive head dims of one row (S = Q K^T contracts
//          over dims).  x8 [rows, d] codes, xs [rows, d/32] scales.
//   V    : blocks of 32 consecutive keys of one head dim (O = P V contracts
//          over keys), stored per 64-key tile transposed as v8t
//          [B*H, T, d, 64] (T = ceil(N/64), keys past N are zero) with the
//          keys of a tile in the order the score accumulators hand them to
//          the P operand: position 32*h + j of a row holds key
//          32*(j/16) + (j%4) + 8*((j%16)/4) + 4*h (h = 0, 1; j = 0..31).
//          vs [B*H, T, 2, 32, d/32]: element (t, b, i, c) scales keys
//          64t + 32b .. +31 of head dim 32c + i.
// Scale rule of a block with largest magnitude amax = m * 2^f (1 <= m < 2):
// X = f - 8 if m <= 1.75 else f - 7 (the smallest X with amax <= 448 * 2^X),
// E = clamp(X + 127, 0, 254), 0 for a zero or subnormal amax; codes are the
// round-to-nearest-even E4M3 values of x * 2^(127 - E).
//
// The attention kernel follows the bf16 one (transposed products, online
// softmax with a lazy offset, K/V tiles streamed by LDS-DMA into two
// buffers of unpadded, XOR-swizzled rows):
//   S^T = K Q^T      v_mfma_scale 32x32x64, K codes from LDS (A), Q codes in
//                    registers (B), their block scales applied by the MFMA;
//   P = exp2(...)    fp32, rounded to E4M3 (values <= 2^8 by the lazy
//                    threshold, so no scale is needed: E8M0 127);
//   l               a ones-operand MFMA over the same rounded P, so the
//                    denominator sees exactly the numerator's weights;
//   O^T += V^T P^T   v_mfma_scale 32x32x64 with the V block scales.
// The fp8 matrix cores run at twice the bf16 rate, so a 64-key tile costs
// nine 32x32x64 products per wave against thirty-two 32x32x16 in bf16.
// d = 128 walks the tiles one per step; d = 64, whose vector work is about
// twice its matrix work, keeps three tiles in flight per step so that the
// two overlap within a wave (FwdF8::walk_pipelined).
// Small grids (a few heads of short sequences) run fwd_fp8_ws_kernel, whose
// four waves split a 32-row block's key tiles between them.
#include <math.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kF8Waves = 4;
constexpr int kF8Threads = 64 * kF8Waves;
constexpr int kF8Keys = 64;              // keys per K/V tile
constexpr float kF8Lazy = 8.0f;          // log2 headroom before a rescale
constexpr int kUnitScale = 0x7F7F7F7F;   // E8M0 127 = 2^0 in every byte

// Scale rule of one block from the float32 bit pattern of its largest
// magnitude: E8M0 exponent E (see the file comment).
__device__ __forceinline__ int mx_scale_exponent(unsigned amax_bits) {
  const int field = (amax_bits >> 23) & 0xFF;
  if (field == 0) return 0;
  const int e = field - 8 + ((amax_bits & 0x7FFFFF) > 0x600000 ? 1 : 0);
  return min(max(e, 0), 254);
}

// x * 2^(127 - E), clamped to the E4M3 range (never binding for finite x),
// two values packed to E4M3 by round to nearest even into bytes 0-1 or 2-3.
__device__ __forceinline__ float mx_scaled(float x, int E) {
  return fminf(fmaxf(__builtin_ldexpf(x, 127 - E), -448.f), 448.f);
}

__device__ __forceinline__ float bf16_to_f32(unsigned short b) { return __uint_as_float((unsigned)b << 16); }

// ------------------------------------------------------------ quantizers
// One thread per 32-element block of a row (Q or K).
template <int D>
__global__ __launch_bounds__(256) void quant_rows_kernel(const unsigned short* __restrict__ x, int64_t rows,
                                                        unsigned char* __restrict__ x8,
                                                        unsigned char* __restrict__ xs) {
  constexpr int NB = D / 32;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * NB) return;
  const unsigned short* src = x + t * 32;
  u32x4 raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = reinterpret_cast<const u32x4*>(src)[i];
  const unsigned short* h = reinterpret_cast<const unsigned short*>(raw);
  unsigned amax = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = max(amax, ((unsigned)h[i] << 16) & 0x7FFFFFFFu);
  const int E = mx_scale_exponent(amax);
  u32x4 out[2];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    int word = 0;
    word = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(bf16_to_f32(h[4 * w]), E),
                                           mx_scaled(bf16_to_f32(h[4 * w + 1]), E), word, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(bf16_to_f32(h[4 * w + 2]), E),
                                           mx_scaled(bf16_to_f32(h[4 * w + 3]), E), word, true);
    out[w / 4][w % 4] = (unsigned)word;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(x8 + t * 32);
  dst[0] = out[0];
  dst[1] = out[1];
  xs[t] = (unsigned char)E;
}

// MX quantization of 32 fp32 values (one block) into 32 E4M3 codes, stored
// as two 16-byte words in element order, and the block's E8M0 scale.
__device__ __forceinline__ unsigned char mx_block32(const float (&val)[32], u32x4 (&out)[2]) {
  unsigned amax = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = max(amax, __float_as_uint(val[i]) & 0x7FFFFFFFu);
  const int E = mx_scale_exponent(amax);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    int word = 0;
    word = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(val[4 * w], E), mx_scaled(val[4 * w + 1], E), word, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(val[4 * w + 2], E), mx_scaled(val[4 * w + 3], E), word, true);
    out[w / 4][w % 4] = (unsigned)word;
  }
  return (unsigned char)E;
}

// Rows of Q or K rotated before quantization (incoherent processing: the
// notes page, section 10 item ③, spreads outlier channels over all head
// dims by an orthogonal transform; QR (KR)^T = Q K^T for orthogonal R).
// Here R = diag(s) H_D with H_D the Sylvester-Hadamard matrix (entries
// +-1, H H^T = D I) and s a sign per head dim, so that
// (Q R)(K R)^T = D Q K^T: the attention on rotated inputs takes scale / D.
// The transform is computed exactly (fp64 butterflies over bf16 inputs; the
// sums stay exact while a row's magnitudes span fewer than 2^38) and rounded
// once to fp32 before the block scales are chosen; an exact zero is taken as
// +0 whatever the signs of the terms that cancelled.  D/64 threads per row
// (adjacent lanes), each holding 64 head dims: at D = 128 the stride-64
// butterfly pairs the two lanes through a shuffle, the rest is in-lane.
template <int D>
__global__ __launch_bounds__(256) void quant_rows_rot_kernel(const unsigned short* __restrict__ x, int64_t rows,
                                                            const signed char* __restrict__ signs,
                                                            unsigned char* __restrict__ x8,
                                                            unsigned char* __restrict__ xs) {
  constexpr int TPR = D / 64;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = t / TPR;
  const int part = (int)(t % TPR);
  if (row >= rows) return;   // both lanes of a row leave together
  const unsigned short* src = x + row * D + 64 * part;
  double v[64];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x4 raw = reinterpret_cast<const u32x4*>(src)[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const unsigned bits = (raw[e / 2] >> (16 * (e % 2))) & 0xFFFFu;
      const int dim = 64 * part + 8 * i + e;
      const double f = (double)__uint_as_float(bits << 16);
      v[8 * i + e] = (signs != nullptr && signs[dim] < 0) ? -f : f;
    }
  }
  if constexpr (TPR == 2) {
    // H_128 = [[H_64, H_64], [H_64, -H_64]]: first (x_lo + x_hi, x_lo - x_hi)
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const double o = __shfl_xor(v[i], 1, 64);
      v[i] = part == 0 ? v[i] + o : o - v[i];
    }
  }
#pragma unroll
  for (int h = 1; h < 64; h *= 2)
#pragma unroll
    for (int i = 0; i < 64; ++i)
      if ((i & h) == 0) {
        const double a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float val[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) val[i] = (float)(v[32 * b + i] + 0.0);   // an exact zero is +0
    u32x4 out[2];
    const unsigned char E = mx_block32(val, out);
    u32x4* dst = reinterpret_cast<u32x4*>(x8 + row * D + 64 * part + 32 * b);
    dst[0] = out[0];
    dst[1] = out[1];
    xs[row * (D / 32) + 2 * part + b] = E;
  }
}

// One workgroup per 256 / (2 D) tiles (64 keys of one head): the tiles'
// key rows are read from HBM as whole 16-byte chunks into LDS, then one
// thread per (tile, key block b, head dim c) takes the 32 keys
// 64t + 32b .. +31 of dim c from LDS.  Their codes go to two 16-byte runs
// of tile row c: positions 16b .. 16b+15 (keys with bit 2 of the key index
// clear) and 32 + 16b .. (bit 2 set), in the accumulator key order.  Keys
// past N read 0.
template <int D>
__global__ __launch_bounds__(256) void quant_v_kernel(const unsigned short* __restrict__ v, int BH, int N,
                                                     int T, unsigned char* __restrict__ v8t,
                                                     unsigned char* __restrict__ vs) {
  constexpr int TPB = 256 / (2 * D);           // tiles per workgroup
  constexpr int CPR = D / 8;                   // 16-byte chunks per key row
  __shared__ __attribute__((aligned(16))) unsigned short rows[TPB * kF8Keys * D];
  const int64_t ntiles = (int64_t)BH * T;
  const int64_t tile0 = (int64_t)blockIdx.x * TPB;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < TPB * kF8Keys * CPR / 256; ++i) {
    const int q = i * 256 + tid;               // chunk of the workgroup's rows
    const int tl = q / (kF8Keys * CPR), key = (q / CPR) % kF8Keys, ch = q % CPR;
    const int64_t tile = tile0 + tl;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (tile < ntiles) {
      const int bh = (int)(tile / T);
      const int kg = (int)(tile % T) * kF8Keys + key;
      if (kg < N) x = *reinterpret_cast<const u32x4*>(v + ((int64_t)bh * N + kg) * D + 8 * ch);
    }
    *reinterpret_cast<u32x4*>(rows + (tl * kF8Keys + key) * D + 8 * ch) = x;
  }
  __syncthreads();
  const int c = tid % D;
  const int b = (tid / D) % 2;
  const int tl = tid / (2 * D);
  const int64_t tile = tile0 + tl;            // bh * T + tile index
  if (tile >= ntiles) return;
  const unsigned short* col = rows + (tl * kF8Keys + 32 * b) * D + c;
  float val[32];
  unsigned amax = 0;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const unsigned short bits = col[r * D];
    val[r] = bf16_to_f32(bits);
    amax = max(amax, ((unsigned)bits << 16) & 0x7FFFFFFFu);
  }
  const int E = mx_scale_exponent(amax);
  // key r of the block (0..31): half h = (r/4)%2, slot j' = (r%4) + 4*(r/8)
  u32x4 run[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // slots j' = 4w .. 4w+3 of half h are keys r = 8w + 4h + 0..3
      const int r0 = 8 * w + 4 * h;
      int word = 0;
      word = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(val[r0], E), mx_scaled(val[r0 + 1], E), word, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(val[r0 + 2], E), mx_scaled(val[r0 + 3], E), word, true);
      run[h][w] = (unsigned)word;
    }
  unsigned char* row = v8t + (tile * D + c) * kF8Keys;
  *reinterpret_cast<u32x4*>(row + 16 * b) = run[0];
  *reinterpret_cast<u32x4*>(row + 32 + 16 * b) = run[1];
  vs[((tile * 2 + b) * 32 + (c % 32)) * (D / 32) + c / 32] = (unsigned char)E;
}

// ---------------------------------------------------------- attention
template <int D> struct F8Cfg {
  // Unpadded LDS rows (every LDS-DMA byte is data); the 16-byte chunks of a
  // row are permuted by an XOR swizzle of the row so that the fragment reads
  // of 16 rows fall in distinct banks: K rows are D bytes (D/16 chunks),
  // V^T rows 64 bytes (4 chunks).
  static constexpr int kStride = D;                    // bytes per K code row in LDS
  static constexpr int vStride = kF8Keys;              // bytes per V^T code row
  static constexpr int kTile = kF8Keys * kStride;      // 8 KB (d=128) or 4 KB (d=64)
  static constexpr int vTile = D * vStride;            // 8 KB or 4 KB
  static constexpr int kDma = kTile / 1024, vDma = vTile / 1024;
  static constexpr int kDmaPerWave = (kDma + kF8Waves - 1) / kF8Waves;
  static constexpr int vDmaPerWave = (vDma + kF8Waves - 1) / kF8Waves;
  static constexpr int KCH = D / 16, VCH = kF8Keys / 16;   // chunks per row
  static_assert(kTile % 1024 == 0 && vTile % 1024 == 0, "tiles must be whole 1 KB blocks");
  // physical chunk = logical chunk ^ swizzle(row)
  static __device__ __forceinline__ int kswz(int r) { return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
  static __device__ __forceinline__ int vswz(int r) { return (r >> 2) & 3; }
};

// Source offset (inside one tile) of LDS-DMA slot `slot` of a tile whose
// rows hold `chunks` 16-byte chunks, swizzled by `swz`.
template <typename SWZ>
__device__ __forceinline__ int f8_dma_offset(int slot, int chunks, SWZ swz) {
  const int r = slot / chunks, pc = slot % chunks;
  return r * 16 * chunks + 16 * (pc ^ swz(r));
}

template <int D, bool CAUSAL>
struct FwdF8 {
  static constexpr int KS = D / 64;          // 64-dim steps of S
  static constexpr int DB = D / 32;          // 32-dim blocks of O
  using C = F8Cfg<D>;

  const unsigned char* kh;     // K codes of the head
  const unsigned char* ksh;    // K scales of the head [N, D/32]
  const unsigned char* vth;    // V^T tiles of the head
  const unsigned char* vsh;    // V scales of the head
  int N, wave, l32, hl, qw, qi;
  float c, thr;
  i32x8 qf[KS];                // Q codes of this lane's query (B operand)
  int qsc;                     // byte ks: scale of Q block 2*ks + hl
  f32x16 acc[DB];              // O^T
  f32x16 lacc;                 // row sums (every element holds the lane's l)
  float m;
  int koff[C::kDmaPerWave], voff[C::vDmaPerWave];
  int k_rd[2 * KS];             // K read offset of chunk 4 ks + 2 h + hl, index 2 ks + h
  int v_rd[2];                 // V^T read offset of chunk 2 hl + h, index h
  unsigned ksw[2][2];          // d = 64: K scale words of the key rows 32kb + l32, per buffer
  unsigned ksel;               // v_perm selector: the scale bytes of blocks hl (and 2 + hl)
  int vs_bytes;                // bytes of the head's V scales (whole tiles)
  unsigned char* kbuf[2];
  unsigned char* vbuf[2];
  // Scale words of the tile per buffer (in the K buffer, after the codes),
  // queued by LDS-DMA with the codes: V (entry l for lane l) and, at
  // d = 128, K (key rows r and 32 + r side by side).
  // Held in registers instead, the words of the next tile were copied
  // between registers across the unrolled loop, and the compiler then
  // waited for every load in flight, the next tile's codes included.
  unsigned char* vsbuf[2];
  unsigned char* ksbuf[2];

  // Queue the K tile at key k0 into buffer B: codes by LDS-DMA, scale words
  // into LDS after the codes (d = 128) or into registers (d = 64).
  template <int B>
  __device__ void issue_k(int k0) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kh + (int64_t)k0 * D), (short)0, (N - k0) * D, 0x00020000);
#pragma unroll
    for (int i = 0; i < C::kDmaPerWave; ++i) {
      const int blk = wave + kF8Waves * i;
      if (C::kDma % kF8Waves == 0 || blk < C::kDma)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kbuf[B] + blk * 1024), 16, koff[i], 0, 0, 0);
    }
    // K scales of keys k0.. (range-checked: keys past N read 0)
    const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(ksh + (int64_t)k0 * (D / 32)), (short)0, (N - k0) * (D / 32), 0x00020000);
    if constexpr (D == 128) {
      // LDS word i holds key row 32 (i % 2) + i / 2, so the two rows a lane
      // reads (l32 and 32 + l32) are one 8-byte read
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rks, (lds_void*)ksbuf[B], 4, 4 * (32 * (l32 & 1) + 16 * hl + (l32 >> 1)), 0, 0, 0);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        ksw[B][kb] = __builtin_amdgcn_raw_buffer_load_b16(rks, 2 * (32 * kb + l32), 0, 0);
    }
#endif
  }

  // Queue the V^T tile at key k0 into buffer B: codes and scale words by
  // LDS-DMA.
  template <int B>
  __device__ void issue_v(int k0) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vth + (int64_t)(k0 / kF8Keys) * D * kF8Keys), (short)0, D * kF8Keys, 0x00020000);
#pragma unroll
    for (int i = 0; i < C::vDmaPerWave; ++i) {
      const int blk = wave + kF8Waves * i;
      if (C::vDma % kF8Waves == 0 || blk < C::vDma)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vbuf[B] + blk * 1024), 16, voff[i], 0, 0, 0);
    }
    // the tile's 64 V scale entries of D/32 bytes, one dword per lane (the
    // range ends with the head's last tile).  Every wave queues the same
    // scale words to the same place: the copies are identical, and a load
    // that depends on the wave would make the compiler wait for every load
    // in flight before each read of LDS.
    const int off = (k0 / kF8Keys) * 64 * (D / 32);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vsh + off), (short)0, vs_bytes - off, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)vsbuf[B], 4, 4 * (32 * hl + l32), 0, 0, 0);
#endif
  }

  // S^T = K Q^T of the K tile in buffer B.
  template <int B>
  __device__ __forceinline__ void scores(f32x16 (&s)[2]) {
    const unsigned char* kt = kbuf[B];
    // d = 128: the scale words of key rows l32 and 32 + l32, adjacent in LDS
    u32x2 kw = {0u, 0u};
    if constexpr (D == 128) kw = reinterpret_cast<const u32x2*>(ksbuf[B])[l32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      // scale word of this lane's key row: byte ks = block 2*ks + hl
      const unsigned w = D == 128 ? kw[kb] : ksw[B][kb];
      const unsigned ksc = __builtin_amdgcn_perm(w, w, ksel);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const unsigned char* src = kt + 32 * kb * C::kStride;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(src + k_rd[2 * ks]);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(src + k_rd[2 * ks + 1]);
        const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        if (ks == 0)
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[ks], s[kb], 0, 0, 0, (int)ksc, 0, qsc);
        else
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[ks], s[kb], 0, 0, 1, (int)ksc, 1, qsc);
      }
    }
  }

  // Causal and tail masks of the tile at key k0, then the row max.
  template <bool MASK>
  __device__ __forceinline__ float masked_max(f32x16 (&s)[2], int k0) {
    if constexpr (MASK) {
      // key = k0 + 32*kb + (r&3) + 8*(r>>2) + 4*hl must be <= min(qi, N-1)
      const int lim = (CAUSAL ? min(qi, N - 1) : N - 1) - k0 - 4 * hl;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + (r & 3) + 8 * (r >> 2) > lim) s[kb][r] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = (kb == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    return max_across_halves(mx);
  }

  // Move the offset to the row max where it passed the offset by more than
  // the lazy headroom, rescaling O and l by exp(m_old - m_new).
  __device__ __forceinline__ void move_offset(float mx, bool upd) {
    const float m_new = upd ? mx : m;
    const float alpha = upd ? __builtin_amdgcn_exp2f((m - m_new) * c) : 1.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) lacc[r] *= alpha;
    m = m_new;
  }

  // P rounded to E4M3 against the current offset: byte 16*kb + r of the
  // operand holds element r of score block kb.
  __device__ __forceinline__ void probs(const f32x16 (&s)[2], i32x8& pf) {
    const float mc = m * c;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * w], c, -mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * w + 1], c, -mc));
        const float p2 = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * w + 2], c, -mc));
        const float p3 = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * w + 3], c, -mc));
        // bytes 0-1 first (bytes 2-3 of the old value are overwritten next,
        // so any register serves as the old value), then bytes 2-3
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, __builtin_bit_cast(int, p0), false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
        pf[4 * kb + w] = word;
      }
  }

  // l += rowsum(P) (a ones-operand product over the rounded P, so the
  // denominator sees exactly the numerator's weights) and O^T += V^T P^T
  // with the V tile in buffer B.
  template <int B>
  __device__ __forceinline__ void pv(const i32x8& pf) {
    const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                        0x38383838, 0x38383838, 0x38383838, 0x38383838};
    lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pf, lacc, 0, 0, 0, kUnitScale, 0, kUnitScale);
    const unsigned char* vt = vbuf[B];
    const int ln = 32 * hl + l32;
    const unsigned vsc = D == 128 ? reinterpret_cast<const unsigned*>(vsbuf[B])[ln]
                                  : reinterpret_cast<const unsigned short*>(vsbuf[B])[ln];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const unsigned char* src = vt + 32 * db * C::vStride;
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(src + v_rd[0]);
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(src + v_rd[1]);
      const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
      if (db == 0)
        acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pf, acc[db], 0, 0, 0, (int)vsc, 0, kUnitScale);
      else if (db == 1)
        acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pf, acc[db], 0, 0, 1, (int)vsc, 0, kUnitScale);
      else if (db == 2)
        acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pf, acc[db], 0, 0, 2, (int)vsc, 0, kUnitScale);
      else
        acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pf, acc[db], 0, 0, 3, (int)vsc, 0, kUnitScale);
    }
  }

  // The end of a step: every load queued in it has landed (the builtin
  // wait, which the compiler sees: it then does not wait for these loads
  // again after the next tile's are queued) and every wave is done with the
  // buffers the next step refills.  A VALU read of a
  // v_mfma_scale_f32_32x32x64_f8f6f4 result needs 20 wait states on the
  // MI355X (measured: at 19 the last result registers still hold their old
  // values), one more than the compiler counts; four wait states after the
  // barrier, which no product may be moved past, keep the first reads of
  // the step's products far enough behind.
  __device__ __forceinline__ void end_step() {
    __builtin_amdgcn_s_waitcnt(0x0070u);   // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 3" ::: "memory");
  }

  // Normalise and store this lane's row: O = O~ / l as bf16, and
  // LSE = scale m + ln l.
  __device__ __forceinline__ void finish(unsigned short* orow, float* lrow, float scale) {
    if (!orow) return;
    const float l_tot = lacc[0];
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = 32 * db + 8 * g + 4 * hl;
        const u32x2 w = {pack_bf16x2(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv),
                         pack_bf16x2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + dim) = w;
      }
    if (lrow) *lrow = m * scale + logf(l_tot);
  }

  // ---- d = 128: one tile per step -------------------------------------
  // Queue tile j + 1 into buffers PAR ^ 1 (it gets the whole step to land),
  // then the scores, softmax and products with V of tile j in buffers PAR.
  // A wave whose last query precedes the tile's first key skips it (causal).
  template <bool MASK, int PAR>
  __device__ void step(int j, int t_end) {
    const int k0 = j * kF8Keys;
    if (j + 1 < t_end) {
      issue_k<PAR ^ 1>(k0 + kF8Keys);
      issue_v<PAR ^ 1>(k0 + kF8Keys);
    }
    if (!MASK || !CAUSAL || k0 <= qw + 31) {
      f32x16 s[2];
      scores<PAR>(s);
      const float mx = masked_max<MASK>(s, k0);
      const bool upd = mx > m + thr;
      if (__builtin_amdgcn_ballot_w64(upd)) {
        asm volatile("" ::: "memory");   // keep this a taken/skipped branch
        move_offset(mx, upd);
      }
      i32x8 pf;
      probs(s, pf);
      pv<PAR>(pf);
    }
    end_step();
  }

  // ---- d = 64: three tiles in flight per step --------------------------
  // At d = 64 a tile's vector work (exponentials, conversions, row max) is
  // about twice its matrix work, so the step overlaps them within the
  // wave: step j multiplies tile j - 1's probabilities with V, takes the
  // scores of tile j + 1 and the softmax of tile j, three independent
  // pieces, with the products placed one by one between runs of the
  // vector work.  The probabilities are taken against the current offset
  // before the offset test; when the row max passes the offset by more
  // than the headroom, O and l are rescaled (after the product with tile
  // j - 1's V, as in the serial order) and the probabilities taken again.
  // Every kept value is the one the serial order gives.
  static constexpr int kProducts = 1 + DB + 2 * KS;   // per step
  static constexpr int kVectorRun = 7;                 // vector instructions after each product

  template <bool MASK>
  __device__ __forceinline__ void softmax_ahead(f32x16 (&s)[2], i32x8& pf, int k0) {
    const float mx = masked_max<MASK>(s, k0);
    probs(s, pf);
    // one product, then two LDS reads (for a later product), then a run of
    // vector instructions (exponentials included), kProducts times
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < kProducts; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, kVectorRun, 0);
    }
    const bool upd = mx > m + thr;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      // The products with V of the previous tile, issued just before, write
      // the accumulators read here: 21 wait states first (see end_step).
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory");
      move_offset(mx, upd);
      probs(s, pf);
    }
  }

  // Step j, PAR = j & 1: queue K of tile j + 2 and V of tile j into buffers
  // PAR; then the product with V of tile j - 1 (probabilities pp, V in
  // buffers PAR ^ 1), the scores of tile j + 1 (K in buffers PAR ^ 1, into
  // sn) and the softmax of tile j (scores sc, probabilities into pc).
  // PREV: tile j - 1 exists; NEXT: tile j + 1 exists.  Every wave does all
  // three (a skipped piece would leave the products' accumulators in
  // different registers on the two paths): the scores of a wave with no
  // query at or after a tile's keys are all masked, its probabilities 0.
  template <bool MASK, int PAR, bool PREV, bool NEXT>
  __device__ void pstep(int j, int t_end, f32x16 (&sc)[2], f32x16 (&sn)[2], const i32x8& pp, i32x8& pc) {
    const int k0 = j * kF8Keys;
    if (j + 2 < t_end) issue_k<PAR>(k0 + 2 * kF8Keys);
    issue_v<PAR>(k0);
    if constexpr (PREV) pv<PAR ^ 1>(pp);
    if constexpr (NEXT) scores<PAR ^ 1>(sn);
    softmax_ahead<MASK>(sc, pc, k0);
    end_step();
  }

  // The product with V of the last tile (buffers B), then 21 wait states
  // before anything reads the accumulators.
  template <int B>
  __device__ void last_pv(const i32x8& pp) {
    pv<B>(pp);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory");
  }

  // The last one or two tiles from tile j on (buffers P first), then the
  // product with V of the last one.
  template <int P>
  __device__ void ptail(int j, int t_end, f32x16 (&sa)[2], f32x16 (&sb)[2], i32x8& pa, i32x8& pb) {
    if (j + 1 < t_end) {
      pstep<true, P, true, true>(j, t_end, sa, sb, pa, pb);
      pstep<true, P ^ 1, true, false>(j + 1, t_end, sb, sa, pb, pa);
      last_pv<P ^ 1>(pa);
    } else {
      pstep<true, P, true, false>(j, t_end, sa, sb, pa, pb);
      last_pv<P>(pb);
    }
  }

  // Tiles [0, full_end) need no mask and have a successor; the one or two
  // after them are diagonal, ragged or last.  FP = full_end & 1 fixes every
  // tile's buffer and register parity at compile time (one copy of the walk
  // per parity: merging the two would leave the accumulators in different
  // registers on the two paths, and the copies then spill).
  template <int FP>
  __device__ __forceinline__ void walk_pipelined(int n_tiles, int full_end, unsigned short* orow, float* lrow, float scale) {
    f32x16 s0[2], s1[2];   // scores of the even and odd tiles
    i32x8 p0, p1;          // their probabilities
    // K of tiles 0 and 1, then the scores of tile 0; the barrier after them
    // frees K buffer 0 for tile 2
    issue_k<0>(0);
    if (n_tiles > 1) issue_k<1>(kF8Keys);
    __builtin_amdgcn_s_waitcnt(0x0070u);   // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    scores<0>(s0);
    __builtin_amdgcn_sched_barrier(0);
    end_step();
    if (FP == 0 && full_end == 0) {         // one or two tiles, both checked
      if (n_tiles > 1) {
        pstep<true, 0, false, true>(0, n_tiles, s0, s1, p1, p0);
        pstep<true, 1, true, false>(1, n_tiles, s1, s0, p0, p1);
        last_pv<1>(p1);
      } else {
        pstep<true, 0, false, false>(0, n_tiles, s0, s1, p1, p0);
        last_pv<0>(p0);
      }
      finish(orow, lrow, scale);
      return;
    }
    pstep<false, 0, false, true>(0, n_tiles, s0, s1, p1, p0);
    int j = 1;
    for (; j + 1 < full_end; j += 2) {
      pstep<false, 1, true, true>(j, n_tiles, s1, s0, p0, p1);
      pstep<false, 0, true, true>(j + 1, n_tiles, s0, s1, p1, p0);
    }
    if constexpr (FP == 0) {
      pstep<false, 1, true, true>(j, n_tiles, s1, s0, p0, p1);
      ++j;
    }
    // j == full_end, of parity FP
    if constexpr (FP == 0) ptail<0>(j, n_tiles, s0, s1, p1, p0);
    else                   ptail<1>(j, n_tiles, s1, s0, p0, p1);
    finish(orow, lrow, scale);
  }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF8Threads, 2) void fwd_fp8_kernel(
    const unsigned char* __restrict__ q8, const unsigned char* __restrict__ qs,
    const unsigned char* __restrict__ k8, const unsigned char* __restrict__ ks,
    const unsigned char* __restrict__ v8t, const unsigned char* __restrict__ vs,
    unsigned short* __restrict__ o, float* __restrict__ lse, int N, int BH, int n_qtiles, float scale,
    int hg, int H, int G) {
  using F = FwdF8<D, CAUSAL>;
  using C = F8Cfg<D>;
  // a K buffer also holds the tile's K and V scale words (256 bytes each)
  // after the codes: the compiler tracks in-flight LDS-DMA per LDS array
  // for a few arrays only, and with more it waits for every load in flight
  // before each read of LDS
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds0[C::kTile + 512];
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds1[C::kTile + 512];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds0[C::vTile];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds1[C::vTile];
  constexpr int BR = 32 * kF8Waves;
  const int T = (N + kF8Keys - 1) / kF8Keys;

  const int tid = threadIdx.x, lane = tid & 63;
  int bh, rank;
  xcd_order(blockIdx.x, BH, n_qtiles, hg, bh, rank);
  const int qt = n_qtiles - 1 - rank;   // heaviest causal tiles first
  const int q0 = qt * BR;

  F f;
  f.kbuf[0] = k_lds0;
  f.kbuf[1] = k_lds1;
  f.vbuf[0] = v_lds0;
  f.vbuf[1] = v_lds1;
  f.ksbuf[0] = k_lds0 + C::kTile;
  f.ksbuf[1] = k_lds1 + C::kTile;
  f.vsbuf[0] = k_lds0 + C::kTile + 256;
  f.vsbuf[1] = k_lds1 + C::kTile + 256;
  // K/V head of this query head (G query heads share one)
  const int64_t kvh = (int64_t)(bh / H) * (H / G) + (bh % H) / G;
  f.kh = k8 + kvh * N * D;
  f.ksh = ks + kvh * N * (D / 32);
  f.vth = v8t + kvh * T * D * kF8Keys;
  f.vsh = vs + kvh * T * 2 * 32 * (D / 32);
  f.vs_bytes = T * 64 * (D / 32);
  f.N = N;
  f.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  f.l32 = lane & 31;
  f.hl = lane >> 5;
  // byte 0 of the K scale operand: block hl of the row; byte 1 (d = 128):
  // block 2 + hl; the rest zero (selector 0x0c)
  f.ksel = D == 128 ? (f.hl ? 0x0c0c0301u : 0x0c0c0200u) : (f.hl ? 0x0c0c0c01u : 0x0c0c0c00u);
  f.qw = q0 + 32 * f.wave;
  f.qi = f.qw + f.l32;
  f.c = scale * kLog2e;
  f.thr = kF8Lazy / f.c;
  f.m = -INFINITY;
#pragma unroll
  for (int db = 0; db < F::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) f.acc[db][r] = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) f.lacc[r] = 0.f;
  // Q codes: bytes 16*hl .. +15 and 32 + 16*hl .. +15 of each 64-dim step
  const bool valid = f.qi < N;
  const int64_t qrow = (int64_t)bh * N + f.qi;
#pragma unroll
  for (int kk = 0; kk < F::KS; ++kk) {
    u32x4 a0 = {0u, 0u, 0u, 0u}, a1 = {0u, 0u, 0u, 0u};
    if (valid) {
      const unsigned char* src = q8 + qrow * D + 64 * kk + 16 * f.hl;
      a0 = *reinterpret_cast<const u32x4*>(src);
      a1 = *reinterpret_cast<const u32x4*>(src + 32);
    }
    f.qf[kk] = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  {
    unsigned w = 0;
    if (valid) {
      if constexpr (D == 128) w = *reinterpret_cast<const unsigned*>(qs + qrow * 4);
      else w = *reinterpret_cast<const unsigned short*>(qs + qrow * 2);
    }
    f.qsc = D == 128 ? (int)(((w >> (8 * f.hl)) & 0xFF) | (((w >> (16 + 8 * f.hl)) & 0xFF) << 8))
                     : (int)((w >> (8 * f.hl)) & 0xFF);
  }
  const auto kswz = [](int r) { return C::kswz(r); };
  const auto vswz = [](int r) { return C::vswz(r); };
#pragma unroll
  for (int i = 0; i < C::kDmaPerWave; ++i)
    f.koff[i] = f8_dma_offset((f.wave + kF8Waves * i) * 64 + lane, C::KCH, kswz);
#pragma unroll
  for (int i = 0; i < C::vDmaPerWave; ++i)
    f.voff[i] = f8_dma_offset((f.wave + kF8Waves * i) * 64 + lane, C::VCH, vswz);
  // K row 32 kb + l32 (the swizzle depends on l32 only), logical chunks
  // 4 ks + hl and 4 ks + 2 + hl; V^T row 32 db + l32, chunks 2 hl, 2 hl + 1
#pragma unroll
  for (int ks = 0; ks < F::KS; ++ks)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      f.k_rd[2 * ks + h] = f.l32 * C::kStride + 16 * ((4 * ks + 2 * h + f.hl) ^ C::kswz(f.l32));
#pragma unroll
  for (int h = 0; h < 2; ++h) f.v_rd[h] = f.l32 * C::vStride + 16 * ((2 * f.hl + h) ^ C::vswz(f.l32));

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int n_tiles = (kv_end + kF8Keys - 1) / kF8Keys;
  const int n_full = CAUSAL ? min(q0 + 1, N) / kF8Keys : N / kF8Keys;

  unsigned short* orow = valid ? o + qrow * D : nullptr;
  float* lrow = (valid && f.hl == 0) ? lse + qrow : nullptr;
  if constexpr (D == 64) {
    const int full_end = min(n_full, n_tiles - 1);
    if (full_end & 1) f.template walk_pipelined<1>(n_tiles, full_end, orow, lrow, scale);
    else              f.template walk_pipelined<0>(n_tiles, full_end, orow, lrow, scale);
  } else {
    // d = 128: one tile per step (the walk is written out here: as a member
    // function the compiler kept the accumulators in two register sets at
    // its exit and spilled)
    f.template issue_k<0>(0);
    f.template issue_v<0>(0);
    __builtin_amdgcn_s_waitcnt(0x0F70u);   // vmcnt(0)
    __syncthreads();
    int j = 0;
    const int full_end = min(n_tiles, n_full);
    for (; j + 1 < full_end; j += 2) {
      f.template step<false, 0>(j, n_tiles);
      f.template step<false, 1>(j + 1, n_tiles);
    }
    if (j < full_end) {
      f.template step<false, 0>(j, n_tiles);
      ++j;
    }
    for (; j < n_tiles; ++j) {
      if (j & 1) f.template step<true, 1>(j, n_tiles);
      else       f.template step<true, 0>(j, n_tiles);
    }
    f.finish(orow, lrow, scale);
  }
}

// ------------------------------------------------------------ small grids
// When the 128-row launch would leave most CUs idle (a few heads of short
// sequences), the time is one workgroup's serial walk over all key tiles.
// Here a workgroup takes 32 query rows and each of its four waves every
// fourth key tile (wave w: tiles w, w+4, ...) through LDS slots of its own,
// so a row's keys are covered by four independent online-softmax passes
// that run side by side; their partial results (offset m, sum l and
// unnormalised O) then meet in LDS and are merged as key chunks are
// (LSE = log sum_w exp(LSE_w); zzszmyf.github.io notes, sections 5 and
// 12.1), each wave writing a quarter of the head dims.  A wave refills its
// K slot with its next tile once the scores have read it and its V slot
// once the product with V has, so each load overlaps the other half of the
// tile's work; the workgroups of a head first touch one share each of the
// head's K and V lines, so that later tiles come from L2.
constexpr int64_t kF8WsMaxGrid = 192;   // 128-row workgroups (3/4 of the CUs)
constexpr int kF8WsMinTiles = 8;

// s_waitcnt immediate: vmcnt n, lgkmcnt and expcnt not waited for (gfx9
// layout: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr unsigned f8_wait_vm(int n) { return 0x0F70u | (unsigned)(n & 15) | ((unsigned)(n >> 4) & 3u) << 14; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF8Threads, 2) void fwd_fp8_ws_kernel(
    const unsigned char* __restrict__ q8, const unsigned char* __restrict__ qs,
    const unsigned char* __restrict__ k8, const unsigned char* __restrict__ ks,
    const unsigned char* __restrict__ v8t, const unsigned char* __restrict__ vs,
    unsigned short* __restrict__ o, float* __restrict__ lse, int N, int BH, int n_qb, float scale,
    int hg, int H, int G) {
  using F = FwdF8<D, CAUSAL>;
  using C = F8Cfg<D>;
  // per wave: a K slot (codes, then the K scale words) and a V slot (codes,
  // then the V scale words); afterwards they hold the wave's partial result
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds[kF8Waves][C::kTile + 256];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds[kF8Waves][C::vTile + 256];
  constexpr int BR = 32;
  constexpr int kDma = C::kDma, vDma = C::vDma;
  constexpr int nK = kDma + (D == 128 ? 1 : 2);   // loads of one K tile (codes, scales)
  constexpr int nV = vDma + 1;                    // loads of one V tile
  const int T = (N + kF8Keys - 1) / kF8Keys;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bh, rank;
  xcd_order(blockIdx.x, BH, n_qb, hg, bh, rank);
  const int q0 = (n_qb - 1 - rank) * BR;   // heaviest causal blocks first

  F f;
  unsigned char* const kt = k_lds[wave];
  unsigned char* const vt = v_lds[wave];
  f.kbuf[0] = kt;
  f.ksbuf[0] = kt + C::kTile;
  f.vbuf[0] = vt;
  f.vsbuf[0] = vt + C::vTile;
  const int64_t kvh = (int64_t)(bh / H) * (H / G) + (bh % H) / G;
  f.kh = k8 + kvh * N * D;
  f.ksh = ks + kvh * N * (D / 32);
  f.vth = v8t + kvh * T * D * kF8Keys;
  f.vsh = vs + kvh * T * 2 * 32 * (D / 32);
  f.vs_bytes = T * 64 * (D / 32);
  f.N = N;
  f.wave = wave;
  f.l32 = lane & 31;
  f.hl = lane >> 5;
  f.ksel = D == 128 ? (f.hl ? 0x0c0c0301u : 0x0c0c0200u) : (f.hl ? 0x0c0c0c01u : 0x0c0c0c00u);
  f.qw = q0;                 // every wave holds the block's 32 rows
  f.qi = q0 + f.l32;
  f.c = scale * kLog2e;
  f.thr = kF8Lazy / f.c;
  f.m = -INFINITY;
#pragma unroll
  for (int db = 0; db < F::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) f.acc[db][r] = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) f.lacc[r] = 0.f;
  const bool valid = f.qi < N;
  const int64_t qrow = (int64_t)bh * N + f.qi;
#pragma unroll
  for (int kk = 0; kk < F::KS; ++kk) {
    u32x4 a0 = {0u, 0u, 0u, 0u}, a1 = {0u, 0u, 0u, 0u};
    if (valid) {
      const unsigned char* src = q8 + qrow * D + 64 * kk + 16 * f.hl;
      a0 = *reinterpret_cast<const u32x4*>(src);
      a1 = *reinterpret_cast<const u32x4*>(src + 32);
    }
    f.qf[kk] = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  {
    unsigned w = 0;
    if (valid) {
      if constexpr (D == 128) w = *reinterpret_cast<const unsigned*>(qs + qrow * 4);
      else w = *reinterpret_cast<const unsigned short*>(qs + qrow * 2);
    }
    f.qsc = D == 128 ? (int)(((w >> (8 * f.hl)) & 0xFF) | (((w >> (16 + 8 * f.hl)) & 0xFF) << 8))
                     : (int)((w >> (8 * f.hl)) & 0xFF);
  }
#pragma unroll
  for (int ks2 = 0; ks2 < F::KS; ++ks2)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      f.k_rd[2 * ks2 + h] = f.l32 * C::kStride + 16 * ((4 * ks2 + 2 * h + f.hl) ^ C::kswz(f.l32));
#pragma unroll
  for (int h = 0; h < 2; ++h) f.v_rd[h] = f.l32 * C::vStride + 16 * ((2 * f.hl + h) ^ C::vswz(f.l32));
  // this wave loads whole tiles: LDS-DMA block i covers 16-byte slots
  // 64 i .. 64 i + 63 of the tile
  const auto kswz = [](int r) { return C::kswz(r); };
  const auto vswz = [](int r) { return C::vswz(r); };
  int koff[kDma], voff[vDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) koff[i] = f8_dma_offset(i * 64 + lane, C::KCH, kswz);
#pragma unroll
  for (int i = 0; i < vDma; ++i) voff[i] = f8_dma_offset(i * 64 + lane, C::VCH, vswz);
  auto load_k = [&](int k0) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(f.kh + (int64_t)k0 * D), (short)0, (N - k0) * D, 0x00020000);
#pragma unroll
    for (int i = 0; i < kDma; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kt + i * 1024), 16, koff[i], 0, 0, 0);
    const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(f.ksh + (int64_t)k0 * (D / 32)), (short)0, (N - k0) * (D / 32), 0x00020000);
    if constexpr (D == 128) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rks, (lds_void*)f.ksbuf[0], 4,
                                               4 * (32 * (f.l32 & 1) + 16 * f.hl + (f.l32 >> 1)), 0, 0, 0);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        f.ksw[0][kb] = __builtin_amdgcn_raw_buffer_load_b16(rks, 2 * (32 * kb + f.l32), 0, 0);
    }
#endif
  };
  auto load_v = [&](int k0) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(f.vth + (int64_t)(k0 / kF8Keys) * D * kF8Keys), (short)0, D * kF8Keys, 0x00020000);
#pragma unroll
    for (int i = 0; i < vDma; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vt + i * 1024), 16, voff[i], 0, 0, 0);
    const int off = (k0 / kF8Keys) * 64 * (D / 32);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(f.vsh + off), (short)0, f.vs_bytes - off, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)f.vsbuf[0], 4, 4 * (32 * f.hl + f.l32), 0, 0, 0);
#endif
  };

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int n_tiles = (kv_end + kF8Keys - 1) / kF8Keys;
  const int n_full = CAUSAL ? min(q0 + 1, N) / kF8Keys : N / kF8Keys;

  // One tile of this wave: its K and V were queued (K first), and loads
  // return in order, so waiting until at most nV (nK) loads are outstanding
  // means that the K (V) loads issued before them have landed.
  auto tile = [&](auto mask, int j) {
    constexpr bool MASK = decltype(mask)::value;
    const int k0 = j * kF8Keys, jn = j + kF8Waves;
    const bool more = jn < n_tiles;
    __builtin_amdgcn_s_waitcnt(f8_wait_vm(nV));
    f32x16 s[2];
    f.template scores<0>(s);
    __builtin_amdgcn_s_waitcnt(0xC07Fu);   // lgkmcnt(0): the K slot has been read
    if (more) load_k(jn * kF8Keys);
    const float mx = f.template masked_max<MASK>(s, k0);
    const bool upd = mx > f.m + f.thr;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      asm volatile("" ::: "memory");   // keep this a taken/skipped branch
      f.move_offset(mx, upd);
    }
    i32x8 pf;
    f.probs(s, pf);
    if (more) __builtin_amdgcn_s_waitcnt(f8_wait_vm(nK));
    else      __builtin_amdgcn_s_waitcnt(f8_wait_vm(0));
    f.template pv<0>(pf);
    __builtin_amdgcn_s_waitcnt(0xC07Fu);   // the V slot has been read
    if (more) load_v(jn * kF8Keys);
  };
  // L2 warm-up: each workgroup of a head touches one share of the head's K
  // code and V code lines (one dword per 128-byte line)
  constexpr int kPrefetch = 2;
  unsigned warm[kPrefetch];
  {
    const int64_t klines = ((int64_t)kv_end * D + 127) / 128;
    const int64_t vlines = ((int64_t)((kv_end + kF8Keys - 1) / kF8Keys) * D * kF8Keys + 127) / 128;
    const int64_t kper = (klines + n_qb - 1) / n_qb, vper = (vlines + n_qb - 1) / n_qb;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)f.kh, (short)0, N * D, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)f.vth, (short)0, T * D * kF8Keys, 0x00020000);
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) {
      const int64_t e = (int64_t)i * kF8Threads + tid;
      warm[i] = 0u;
      if (e < kper) {
        const int64_t line = (int64_t)rank * kper + e;
        if (line < klines) warm[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, (int)(line * 128), 0, 0);
      } else if (e < kper + vper) {
        const int64_t line = (int64_t)rank * vper + (e - kper);
        if (line < vlines) warm[i] = __builtin_amdgcn_raw_buffer_load_b32(rv, (int)(line * 128), 0, 0);
      }
    }
  }
  int j = wave;
  if (j < n_tiles) {
    load_k(j * kF8Keys);
    load_v(j * kF8Keys);
    for (; j < min(n_full, n_tiles); j += kF8Waves) tile(std::false_type{}, j);
    for (; j < n_tiles; j += kF8Waves) tile(std::true_type{}, j);
  }
  {
    unsigned x = 0u;
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) x ^= warm[i];
    asm volatile("" ::"v"(x));
  }
  __builtin_amdgcn_s_waitcnt(0x0070u);   // vmcnt(0) lgkmcnt(0)
  // 21 wait states before the accumulators of the last products are read
  // (a VALU read of a v_mfma_scale_f32_32x32x64_f8f6f4 result needs 20)
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory");
  __syncthreads();

  // Partial results to LDS: the unnormalised O^T of the wave as fp32
  // [32 rows][D/2] per half of the head dims, the first half in its K slot
  // and the second in its V slot (16-byte chunk c of a row at c ^ (row mod
  // D/8)), its offsets and row sums after them.
  constexpr int HC = D / 8;   // 16-byte chunks per row of a half
  {
#pragma unroll
    for (int db = 0; db < F::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 8 * db + 2 * g + f.hl;    // chunk of dims 32 db + 8 g + 4 hl
        float* ob = reinterpret_cast<float*>(c < HC ? kt : vt);
        const float4 w = {f.acc[db][4 * g], f.acc[db][4 * g + 1], f.acc[db][4 * g + 2], f.acc[db][4 * g + 3]};
        *reinterpret_cast<float4*>(ob + f.l32 * (D / 2) + 4 * ((c % HC) ^ (f.l32 % HC))) = w;
      }
    if (f.hl == 0) {
      reinterpret_cast<float*>(kt + C::kTile)[f.l32] = f.m;
      reinterpret_cast<float*>(vt + C::vTile)[f.l32] = f.lacc[0];
    }
  }
  __syncthreads();

  // Merge: wave w writes head dims [w D/4, (w+1) D/4) of the 32 rows; lane
  // (row, half) takes D/8 of them.  Key 0 is visible to every row and sits
  // in wave 0's first tile, so the row max M is finite; a wave that saw no
  // key of a row (offset -inf) weighs 0.
  const int row = lane & 31, hh = lane >> 5;
  constexpr int NC = D / 32;                   // 16-byte chunks per lane
  float mw[kF8Waves], M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kF8Waves; ++w) {
    mw[w] = reinterpret_cast<const float*>(k_lds[w] + C::kTile)[row];
    M = fmaxf(M, mw[w]);
  }
  float L = 0.f;
  float out[4 * NC];
#pragma unroll
  for (int e = 0; e < 4 * NC; ++e) out[e] = 0.f;
  const int c0 = wave * (D / 16) + hh * NC;   // first chunk of this lane
#pragma unroll
  for (int w = 0; w < kF8Waves; ++w) {
    const float a = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mw[w] - M) * f.c);
    L += a * reinterpret_cast<const float*>(v_lds[w] + C::vTile)[row];
    const float* ob = reinterpret_cast<const float*>(c0 < HC ? k_lds[w] : v_lds[w]);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int cc = (c0 + c) % HC;
      const float4 x = *reinterpret_cast<const float4*>(ob + row * (D / 2) + 4 * (cc ^ (row % HC)));
      out[4 * c] += a * x.x;
      out[4 * c + 1] += a * x.y;
      out[4 * c + 2] += a * x.z;
      out[4 * c + 3] += a * x.w;
    }
  }
  if (q0 + row >= N) return;
  const int64_t grow = (int64_t)bh * N + q0 + row;
  const float inv = 1.f / L;
  unsigned short* orow = o + grow * D + 4 * c0;
#pragma unroll
  for (int c = 0; c < NC; c += 2) {
    const u32x4 w = {pack_bf16x2(out[4 * c] * inv, out[4 * c + 1] * inv),
                     pack_bf16x2(out[4 * c + 2] * inv, out[4 * c + 3] * inv),
                     pack_bf16x2(out[4 * c + 4] * inv, out[4 * c + 5] * inv),
                     pack_bf16x2(out[4 * c + 6] * inv, out[4 * c + 7] * inv)};
    *reinterpret_cast<u32x4*>(orow + 4 * c) = w;
  }
  if (wave == 0 && hh == 0) lse[grow] = M * scale + logf(L);
}

template <int D>
hipError_t launch_quant_rows(const void* x, int64_t rows, void* x8, void* xs, hipStream_t stream) {
  const int64_t threads = rows * (D / 32);
  hipLaunchKernelGGL((quant_rows_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const unsigned short*>(x), rows, static_cast<unsigned char*>(x8),
                     static_cast<unsigned char*>(xs));
  return hipGetLastError();
}

template <int D>
hipError_t launch_quant_rows_rot(const void* x, int64_t rows, const void* signs, void* x8, void* xs,
                                 hipStream_t stream) {
  const int64_t threads = rows * (D / 64);
  hipLaunchKernelGGL((quant_rows_rot_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const unsigned short*>(x), rows, static_cast<const signed char*>(signs),
                     static_cast<unsigned char*>(x8), static_cast<unsigned char*>(xs));
  return hipGetLastError();
}

template <int D>
hipError_t launch_quant_v(const void* v, int BH, int N, void* v8t, void* vs, hipStream_t stream) {
  const int T = (N + kF8Keys - 1) / kF8Keys;
  const int64_t tiles = (int64_t)BH * T;
  constexpr int TPB = 256 / (2 * D);
  hipLaunchKernelGGL((quant_v_kernel<D>), dim3((unsigned)((tiles + TPB - 1) / TPB)), dim3(256), 0, stream,
                     static_cast<const unsigned short*>(v), BH, N, T, static_cast<unsigned char*>(v8t),
                     static_cast<unsigned char*>(vs));
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_fp8(const Fp8Problem& p, hipStream_t stream) {
  const int BH = p.B * p.H;
  const int n_qtiles = (p.N + 32 * kF8Waves - 1) / (32 * kF8Waves);
  if ((int64_t)n_qtiles * BH <= kF8WsMaxGrid && (p.N + kF8Keys - 1) / kF8Keys >= kF8WsMinTiles) {
    const int n_qb = (p.N + 31) / 32;
    hipLaunchKernelGGL((fwd_fp8_ws_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)n_qb * BH)), dim3(kF8Threads), 0,
                       stream, static_cast<const unsigned char*>(p.q8), static_cast<const unsigned char*>(p.qs),
                       static_cast<const unsigned char*>(p.k8), static_cast<const unsigned char*>(p.ks),
                       static_cast<const unsigned char*>(p.v8t), static_cast<const unsigned char*>(p.vs),
                       static_cast<unsigned short*>(p.o), p.lse, p.N, BH, n_qb, p.scale,
                       xcd_head_group(BH, n_qb, 1, CAUSAL ? n_qb : 0, 1, 4), p.H, p.H / p.Hkv);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)n_qtiles * BH)),
                     dim3(kF8Threads), 0, stream, static_cast<const unsigned char*>(p.q8),
                     static_cast<const unsigned char*>(p.qs), static_cast<const unsigned char*>(p.k8),
                     static_cast<const unsigned char*>(p.ks), static_cast<const unsigned char*>(p.v8t),
                     static_cast<const unsigned char*>(p.vs), static_cast<unsigned short*>(p.o), p.lse, p.N,
                     BH, n_qtiles, p.scale, xcd_head_group(BH, n_qtiles, 1, CAUSAL ? n_qtiles : 0, 1, 4),
                     p.H, p.H / p.Hkv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_qk_fp8(const void* x, int64_t rows, int d, void* x8, void* xs, hipStream_t stream) {
  return d == 64 ? launch_quant_rows<64>(x, rows, x8, xs, stream) : launch_quant_rows<128>(x, rows, x8, xs, stream);
}

hipError_t launch_quantize_qk_fp8_rotated(const void* x, int64_t rows, int d, const void* signs, void* x8,
                                          void* xs, hipStream_t stream) {
  return d == 64 ? launch_quant_rows_rot<64>(x, rows, signs, x8, xs, stream)
                 : launch_quant_rows_rot<128>(x, rows, signs, x8, xs, stream);
}

hipError_t launch_quantize_v_fp8(const void* v, int BH, int N, int d, void* v8t, void* vs, hipStream_t stream) {
  return d == 64 ? launch_quant_v<64>(v, BH, N, v8t, vs, stream) : launch_quant_v<128>(v, BH, N, v8t, vs, stream);
}

hipError_t launch_fwd_fp8(const Fp8Problem& p, hipStream_t stream) {
  if (p.d == 64) return p.causal ? launch_fp8<64, true>(p, stream) : launch_fp8<64, false>(p, stream);
  return p.causal ? launch_fp8<128, true>(p, stream) : launch_fp8<128, false>(p, stream);
}

}  // namespace fa
