// bf16 attention forward on the gfx950 matrix cores.
//
// One workgroup owns 128 (or 256) query rows of one (batch, head) and streams the K/V
// tiles of that head through LDS; the scores and probabilities of a tile live
// only in registers and are merged into a running row max m, row sum l and an
// unnormalised fp32 accumulator, which is rescaled by exp(m_old - m_new) when
// the max moves and divided by l once at the end (aiqz.cc Flash Attention IO
// article, sections 分块Tiling策略 and 在线Softmax算法; cf-1.com FlashAttention
// write-up, sections 3.2 and 4.3).  Queries are the outer loop and keys the
// inner one, so a query tile reads Q once and writes O once.
//
// Work inside a workgroup (4 waves of 64 lanes, 32 query rows per wave, or
// two blocks of 32 when d = 64 and the grid is large; see launch):
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
// LDS rows are unpadded (2*D bytes, so every LDS-DMA byte is data): the
// 16-byte chunks of each row are permuted by an XOR swizzle of the row, set
// when the DMA source offsets are chosen, so that the K fragment reads of 16
// rows and the transposed V reads of 4 rows fall in distinct banks.  A
// lane's read addresses are then one register per K k-step and per V
// head-dim block, plus compile-time offsets.
// Rescaling is lazy and needs no row max on most tiles: a tile's
// probabilities are first taken against the current offset m; they are kept
// when no lane's share of their sum exceeds 2^48 (so no probability does
// either).  Only otherwise (a row's first tile, where m = -inf, or a score far
// above m) is the row max taken, m moved to it, the accumulator rescaled by
// exp(m_old - m_new) and the probabilities redone.  Since O and l share the
// offset the result is unchanged (the softmax identity holds for any offset;
// zzszmyf.github.io notes, section 5.1).
// Causal: key tiles wholly above the diagonal are never loaded, masking is
// applied only on diagonal tiles and on the ragged last tile.
// Grouped K/V heads (MQA/GQA, the K/V-read saving named in the aiqz.cc
// article's tuning section): the G query heads that share one K/V head are
// adjacent in [B, H, Nq, d], so a K/V head's queries form one contiguous
// block of G*Nq rows; row r of it sits at position r % Nq of its head.  A
// workgroup's 128 rows are taken from that block, either one head at a time
// (long causal heads, so the heaviest tiles can go first) or packed across
// heads (short or non-causal heads: decoding with G heads reads K/V once).
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// s_waitcnt immediates (gfx9 layout: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8; a field at its maximum does not wait)
constexpr unsigned wait_vm(int n) { return 0x0F70u | (unsigned)(n & 15) | ((unsigned)(n >> 4) & 3u) << 14; }
constexpr unsigned kWaitVm0 = wait_vm(0);
constexpr unsigned kWaitLgkm0 = 0xC07Fu;
constexpr unsigned kWaitVm0Lgkm0 = 0x0070u;
constexpr int kKeys = 64;                 // keys per K/V tile (Bc)
// A tile's probabilities against a stale offset are kept while every lane's
// share of their sum (32 of them) is at most this, so no kept probability
// exceeds 2^48: with fewer than 2^31 keys the accumulators stay below
// 2^79 max|v|, far from the fp32 range limit for any V a bf16 caller has
// short of 2^49.
constexpr float kProbSumMax = 0x1p48f;

template <int D> struct Cfg {
  // Rows are stored unpadded (2*D bytes); each row's 16-byte chunks are
  // permuted by an XOR swizzle so that fragment reads stay conflict-free.
  static constexpr int kStride = 2 * D;                // bytes per K row
  static constexpr int vStride = 2 * D;                // bytes per V row
  static constexpr int kTile = kKeys * kStride;        // bytes of one K tile
  static constexpr int vTile = kKeys * vStride;        // bytes of one V tile
  static constexpr int lds = 2 * (kTile + vTile);      // two K and two V buffers
  static constexpr int kDma = kTile / 1024;            // 1 KB LDS-DMA loads per tile
  static constexpr int vDma = vTile / 1024;
  static constexpr int kDmaPerWave = (kDma + kWaves - 1) / kWaves;
  static constexpr int vDmaPerWave = (vDma + kWaves - 1) / kWaves;
  static constexpr int CH = D / 8;                     // 16-byte chunks per row
  // physical chunk = logical chunk ^ swizzle(row)
  static __device__ __forceinline__ int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  static __device__ __forceinline__ int vswz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// SPLIT: the workgroup covers one chunk of the keys and may meet rows that
// have no valid key in it; such rows keep m = -inf and l = 0.
template <int D, int QB, bool CAUSAL, bool SPLIT>
struct Fwd {
  static constexpr int KS = D / 16, DB = D / 32, KB = kKeys / 32, PS = kKeys / 16;
  static constexpr int WR = 32 * QB;        // query rows per wave

  const unsigned short* kh;
  const unsigned short* vh;
  int N;                  // keys (Nk)
  int coff;               // causal offset Nk - Nq: query i sees keys j <= i + coff
  int wave, l32, hl;
  int pos[QB];            // position inside its head of this lane's query, per block
  int wlast;              // causal: last key any valid query of this wave sees (-1: none)
  bool rows;              // the wave has a valid query row
  float c;                // scale * log2(e)
  bf16x8 qf[QB][KS];      // Q fragments (B operand of S^T = K Q^T), per 32-row block
  f32x16 acc[QB][DB];     // O^T accumulators: lane holds query l%32 of each block
  float m[QB];            // exponent offsets (raw-score units)
  float l[QB];            // this lane's share of the row sums, relative to m
  int koff[Cfg<D>::kDmaPerWave];   // source byte offsets of the K LDS-DMA slots
  int voff[Cfg<D>::vDmaPerWave];   // source byte offsets of the V LDS-DMA slots
  int k_rd[KS];                    // this lane's K fragment read offset for each k-step
  int v_rd[DB];                    // this lane's V fragment read offset for each head-dim block
  // LDS: K and V of two tiles, as four separate arrays selected at compile
  // time, so the compiler sees that the LDS-DMA writes into one buffer do not
  // touch the buffers being read and inserts no wait for them.
  unsigned char* kbuf[2];
  unsigned char* vbuf[2];

  __device__ void setup_offsets(int lane) {
    // LDS-DMA slot (16 bytes) -> source: row = slot / CH, physical chunk =
    // slot % CH holds logical chunk physical ^ swizzle(row)
#pragma unroll
    for (int i = 0; i < Cfg<D>::kDmaPerWave; ++i) {
      const int slot = (wave + kWaves * i) * 64 + lane;
      const int r = slot / Cfg<D>::CH, pc = slot % Cfg<D>::CH;
      koff[i] = r * (2 * D) + 16 * (pc ^ Cfg<D>::kswz(r));
    }
#pragma unroll
    for (int i = 0; i < Cfg<D>::vDmaPerWave; ++i) {
      const int slot = (wave + kWaves * i) * 64 + lane;
      const int r = slot / Cfg<D>::CH, pc = slot % Cfg<D>::CH;
      voff[i] = r * (2 * D) + 16 * (pc ^ Cfg<D>::vswz(r));
    }
    // K fragment of k-step ks: row l32 (+32 kb), logical chunk 2 ks + hl
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      k_rd[ks] = l32 * Cfg<D>::kStride + 16 * ((2 * ks + hl) ^ Cfg<D>::kswz(l32));
    // Transposed V reads: in each 16-lane group g, lane 4e + j addresses key
    // row 4*(g/2) + e (+8, +16 ps: the swizzle is unchanged) and head dims
    // 16*(g%2) + 4j .. +3 of 32-dim block db, i.e. logical chunk
    // 4 db + 2 (g%2) + j/2, byte 8 (j%2) within it.
    const int g = lane >> 4, e = (lane >> 2) & 3, j = lane & 3;
    const int vr = 4 * (g >> 1) + e;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      v_rd[db] = vr * Cfg<D>::vStride + 16 * ((4 * db + 2 * (g & 1) + (j >> 1)) ^ Cfg<D>::vswz(vr)) + 8 * (j & 1);
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

  // Probabilities of one 32-row block against the offset mc = m*c, rounded
  // to bf16 for the product, and this lane's share of their sum, taken over
  // the same rounded values (two per v_dot2_f32_bf16) so numerator and
  // denominator see identical weights.  The dot2 takes the converted pair
  // itself: taking it from an element of the vector under construction is
  // miscompiled (the same element is summed repeatedly).
  __device__ __forceinline__ float probs(const f32x16 (&s)[KB], bf16x8 (&pf)[PS], float mc) {
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
          const bf16x2 pb = __builtin_convertvector((f32x2{p0, p1}), bf16x2);
          if (e & 2) ps1 = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, ps1, false);
          else       ps0 = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, ps0, false);
          w[e / 2] = __builtin_bit_cast(unsigned, pb);
        }
        pf[2 * kb + half] = __builtin_bit_cast(bf16x8, w);
      }
    return ps0 + ps1;
  }

  // Online-softmax step of one 32-row block for the tile at key k0: writes
  // the bf16 probabilities, moving the offset (and rescaling) when needed,
  // and adds their row sum.  FIRST: the wave's first tile, whose offset is
  // still -inf, goes straight to the row max.
  template <bool MASK, bool FIRST = false>
  __device__ __forceinline__ void softmax(int qb, f32x16 (&s)[KB], bf16x8 (&pf)[PS], int k0) {
    if constexpr (MASK) {
      // key = k0 + 32*kb + (r&3) + 8*(r>>2) + 4*hl must be <= min(qi+coff, N-1)
      const int lim = (CAUSAL ? min(pos[qb] + coff, N - 1) : N - 1) - k0 - 4 * hl;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + (r & 3) + 8 * (r >> 2) > lim) s[kb][r] = -INFINITY;
    }
    // Probabilities against the current offset, kept unless some lane's
    // share of their sum is above kProbSumMax or NaN (m = -inf on a row's
    // first tile gives inf or NaN); then the offset moves to the row max
    // (wave-uniform branch; rows whose max did not rise keep alpha = 1) and
    // they are redone.
    float ps = 0.f;
    if (!FIRST) ps = probs(s, pf, m[qb] * c);
    if (FIRST || __builtin_amdgcn_ballot_w64(!(ps <= kProbSumMax))) {
      asm volatile("" ::: "memory");
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = (kb == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = max_across_halves(mx);
      const bool upd = mx > m[qb];
      const float m_new = upd ? mx : m[qb];
      const float alpha = upd ? __builtin_amdgcn_exp2f((m[qb] - m_new) * c) : 1.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
      l[qb] *= alpha;
      m[qb] = m_new;
      // a key-split chunk can hold no valid key for a row (m still -inf):
      // its probabilities must come out 0, not exp2(-inf + inf)
      const float mc = (SPLIT && m_new == -INFINITY) ? 0.f : m_new * c;
      ps = probs(s, pf, mc);
    }
    l[qb] += ps;
  }

  // S^T = K Q^T of the tile whose K sits at kt, for every block (each K
  // fragment feeds all blocks).
  __device__ __forceinline__ void scores(const unsigned char* kt, f32x16 (&s)[QB][KB]) {
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
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt + k_rd[ks] + 32 * kb * Cfg<D>::kStride);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ks], s[qb][kb], 0, 0, 0);
      }
  }

  // O^T += V^T P^T with V of the tile at vt (each V fragment feeds all blocks).
  __device__ __forceinline__ void pv(const unsigned char* vt, const bf16x8 (&pf)[QB][PS]) {
#pragma unroll
    for (int ps = 0; ps < PS; ++ps)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const unsigned char* src = vt + v_rd[db] + 16 * ps * Cfg<D>::vStride;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + 8 * Cfg<D>::vStride));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][ps], acc[qb][db], 0, 0, 0);
      }
  }

  // Consume the tile in buffers PAR: the scores, the softmax merges, then
  // the product with V.
  template <bool MASK, int PAR, bool FIRST = false>
  __device__ __forceinline__ void consume(int k0) {
    f32x16 s[QB][KB];
    scores(kbuf[PAR], s);
    bf16x8 pf[QB][PS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) softmax<MASK, FIRST>(qb, s[qb], pf[qb], k0);
    pv(vbuf[PAR], pf);
  }

  // One pipeline step: queue tile j+1 into the other buffers (it gets the
  // whole step to land), consume tile j, wait and synchronise.
  // PAR = j & 1 selects the buffers at compile time; FIRST marks the
  // workgroup's first tile.
  template <bool MASK, int PAR, bool FIRST = false>
  __device__ void step(int j, int t_end) {
    const int k0 = j * kKeys;
    if (j + 1 < t_end) {
      issue<false, PAR ^ 1>(k0 + kKeys);
      issue<true, PAR ^ 1>(k0 + kKeys);
    }
    // Causal: a wave whose last query precedes the tile's first key has
    // nothing to do here or later; key chunks of a decoding step leave whole
    // waves without a query row.  The barrier below stays unconditional.
    if ((!SPLIT || rows) && (!MASK || !CAUSAL || k0 <= wlast)) consume<MASK, PAR, FIRST>(k0);
    // The builtin wait, not inline assembly: the compiler then knows that
    // every load before it has landed, and does not wait for them again
    // after the next tile's loads are queued (which would wait for those too).
    __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
    __builtin_amdgcn_s_barrier();
  }
};

// Positions covered by rows [a, a + n) (n >= 1) of a K/V head's query block
// (row r is position r % Nq): one run when the rows stay inside one head,
// else every position of a head.
__device__ __forceinline__ void position_range(int a, int n, int Nq, int& lo, int& hi) {
  const int p0 = a % Nq;
  if (p0 + n - 1 < Nq) {
    lo = p0;
    hi = p0 + n - 1;
  } else {
    lo = 0;
    hi = Nq - 1;
  }
}

// One workgroup per (query tile, key chunk, batch * K/V head).  The query
// rows of K/V head bkv are rows [bkv*G*Nq, (bkv+1)*G*Nq) of Q, O and LSE.
// Blocks map to heads and tiles through xcd_order with hg heads per group.
// tph > 0: tiles stay inside one query head (tph tiles per head, G heads);
// tph == 0: tiles are packed over the whole block of G*Nq rows.  Without
// SPLIT the single chunk is every key and O/LSE are written directly; with
// SPLIT the chunk's own normalised O (fp32) and LSE go to opart/lpart for
// the merge.
template <int D, int QB, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(kThreads, (QB == 1 || D == 64) ? 2 : 1) void fwd_bf16_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
    const unsigned short* __restrict__ v, unsigned short* __restrict__ o,
    float* __restrict__ lse, int Nq, int Nk, int G, int BHkv, int n_qtiles, int tph,
    float scale, int splits, float* __restrict__ opart, float* __restrict__ lpart, int hg) {
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds0[Cfg<D>::kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds1[Cfg<D>::kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds0[Cfg<D>::vTile];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds1[Cfg<D>::vTile];
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int BR = 32 * QB * kWaves;   // query rows per workgroup
  using F = Fwd<D, QB, CAUSAL, SPLIT>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Heaviest query tiles first (causal work grows with the position).
  int bkv, rest;   // K/V head and rank of the tile (and chunk) within it
  xcd_order(blockIdx.x, BHkv, (SPLIT ? splits : 1) * n_qtiles, hg, bkv, rest);
  const int split = SPLIT ? rest % splits : 0;
  const int idx = SPLIT ? rest / splits : rest;
  const int R = G * Nq;                  // query rows per K/V head
  int r0, nr;                            // this tile: rows [r0, r0 + nr) of the block
  if (tph == 0) {
    r0 = (n_qtiles - 1 - idx) * BR;
    nr = min(BR, R - r0);
  } else {
    const int pt = tph - 1 - idx / G;
    r0 = (idx % G) * Nq + pt * BR;
    nr = min(BR, Nq - pt * BR);
  }
  const int64_t qblock = (int64_t)bkv * R;   // first Q/O/LSE row of the block
  const int64_t khead = (int64_t)bkv * Nk * D;

  F f;
  f.kbuf[0] = k_lds0;
  f.kbuf[1] = k_lds1;
  f.vbuf[0] = v_lds0;
  f.vbuf[1] = v_lds1;
  f.kh = k + khead;
  f.vh = v + khead;
  f.N = Nk;
  f.coff = Nk - Nq;
  f.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  f.l32 = lane & 31;
  f.hl = lane >> 5;
  {
    const int w0 = f.wave * F::WR;       // first row of this wave in the tile
    int lo, hi;
    f.rows = w0 < nr;
    if (w0 < nr) {
      position_range(r0 + w0, min(F::WR, nr - w0), Nq, lo, hi);
      f.wlast = hi + f.coff;
    } else {
      f.wlast = -1;
    }
  }
  f.c = scale * kLog2e;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    f.m[qb] = -INFINITY;
    f.l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) f.acc[qb][db][r] = 0.f;
    const int lr = f.wave * F::WR + 32 * qb + f.l32;   // row inside the tile
    f.pos[qb] = (r0 + lr) % Nq;
    const unsigned short* qrow = q + (qblock + r0 + lr) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (lr < nr) raw = *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * f.hl);
      f.qf[qb][ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  f.setup_offsets(lane);

  // Key tiles this workgroup's rows need, and its chunk [t0, t1) of them.
  int pmin, pmax;
  position_range(r0, nr, Nq, pmin, pmax);
  const int kv_end = CAUSAL ? min(Nk, pmax + 1 + f.coff) : Nk;
  const int n_tiles = (kv_end + kKeys - 1) / kKeys;
  const int t0 = SPLIT ? (int)((int64_t)split * n_tiles / splits) : 0;
  const int t1 = SPLIT ? (int)((int64_t)(split + 1) * n_tiles / splits) : n_tiles;
  // Tiles before n_full need no mask: every key is < Nk and, when causal,
  // visible to the workgroup's earliest query.
  const int n_full = CAUSAL ? min(pmin + f.coff + 1, Nk) / kKeys : Nk / kKeys;

  if (t0 < t1) {
    f.template issue<false, 0>(t0 * kKeys);
    f.template issue<true, 0>(t0 * kKeys);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    // buffer parity counts from t0.  The first tile goes straight to the
    // row max (the offset is still -inf), skipping the probability pass that
    // would be discarded.
    int j = t0;
    const int full_end = max(t0, min(t1, n_full));
    if (j < full_end) f.template step<false, 0, true>(j, t1);
    else              f.template step<true, 0, true>(j, t1);
    ++j;
    for (; j + 1 < full_end; j += 2) {
      f.template step<false, 1>(j, t1);
      f.template step<false, 0>(j + 1, t1);
    }
    if (j < full_end) {
      f.template step<false, 1>(j, t1);
      ++j;
    }
    for (; j < t1; ++j) {
      if ((j - t0) & 1) f.template step<true, 1>(j, t1);
      else              f.template step<true, 0>(j, t1);
    }
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = sum_across_halves(f.l[qb]);
    const int lr = f.wave * F::WR + 32 * qb + f.l32;
    if (lr >= nr) continue;
    const int64_t row = qblock + r0 + lr;
    if constexpr (!SPLIT) {
      // O = acc / l in bf16 (round to nearest even), LSE = scale*m + ln l.
      const float inv = 1.f / l_tot;
      unsigned short* orow = o + row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dim = 32 * db + 8 * g + 4 * f.hl;
          const u32x2 w = {pack_bf16x2(f.acc[qb][db][4 * g] * inv, f.acc[qb][db][4 * g + 1] * inv),
                           pack_bf16x2(f.acc[qb][db][4 * g + 2] * inv, f.acc[qb][db][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + dim) = w;
        }
      if (f.hl == 0) lse[row] = f.m[qb] * scale + logf(l_tot);
    } else {
      // this chunk's normalised O and LSE; a row with no valid key in the
      // chunk gets O = 0 and LSE = -inf (weight 0 in the merge)
      const bool empty = !(l_tot > 0.f);
      const float inv = empty ? 0.f : 1.f / l_tot;
      const int64_t prow = (int64_t)split * BHkv * R + row;
      float* orow = opart + prow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dim = 32 * db + 8 * g + 4 * f.hl;
          const float4 w = {f.acc[qb][db][4 * g] * inv, f.acc[qb][db][4 * g + 1] * inv,
                            f.acc[qb][db][4 * g + 2] * inv, f.acc[qb][db][4 * g + 3] * inv};
          *reinterpret_cast<float4*>(orow + dim) = w;
        }
      if (f.hl == 0) lpart[prow] = empty ? -INFINITY : f.m[qb] * scale + logf(l_tot);
    }
  }
}

// Small grids: one workgroup per 32 query rows, its four waves splitting
// the keys.  When ceil(rows/128) workgroups of the kernel above would leave
// most CUs idle (a few heads of short sequences), the time is one
// workgroup's serial walk over all key tiles.  Here every wave holds the
// same 32 rows and takes every fourth key tile (wave w: tiles w, w+4, ...)
// through LDS slots of its own, so a row's keys are covered by four
// independent online-softmax passes that run side by side; the four partial
// results (offset m, sum l and unnormalised O of each wave) then meet in LDS
// and are merged as chunks are (LSE = log sum_w exp(LSE_w); notes page,
// sections 5 and 12.1), each wave writing a quarter of the head dims.
// A wave's K slot is refilled with its next tile's keys as soon as the
// scores have read it, and the V slot once the product with V has, so each
// load overlaps the other half of the tile's work.  A wave's first tile goes
// straight to the row max (its offset is still -inf), and the workgroups of
// a head first touch one share each of the head's K and V lines, so that
// later tiles come from L2.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void fwd_bf16_ws_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
    const unsigned short* __restrict__ v, unsigned short* __restrict__ o,
    float* __restrict__ lse, int Nq, int Nk, int G, int BHkv, int n_qtiles, int tph,
    float scale, int hg) {
  // per wave: one K and one V tile (separate arrays, so that the compiler
  // sees that V loads in flight do not touch K and the other way round)
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds[kWaves][Cfg<D>::kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds[kWaves][Cfg<D>::vTile];
  constexpr int KS = D / 16, DB = D / 32, BR = 32;
  constexpr int kDma = Cfg<D>::kDma, vDma = Cfg<D>::vDma;
  using F = Fwd<D, 1, CAUSAL, true>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bkv, idx;
  xcd_order(blockIdx.x, BHkv, n_qtiles, hg, bkv, idx);
  const int R = G * Nq;
  int r0, nr;
  if (tph == 0) {
    r0 = (n_qtiles - 1 - idx) * BR;
    nr = min(BR, R - r0);
  } else {
    const int pt = tph - 1 - idx / G;
    r0 = (idx % G) * Nq + pt * BR;
    nr = min(BR, Nq - pt * BR);
  }
  const int64_t qblock = (int64_t)bkv * R;
  const int64_t khead = (int64_t)bkv * Nk * D;

  F f;
  unsigned char* const kt = k_lds[wave];
  unsigned char* const vt = v_lds[wave];
  f.kh = k + khead;
  f.vh = v + khead;
  f.N = Nk;
  f.coff = Nk - Nq;
  f.wave = wave;
  f.l32 = lane & 31;
  f.hl = lane >> 5;
  f.rows = true;
  int pmin, pmax;
  position_range(r0, nr, Nq, pmin, pmax);
  f.wlast = pmax + f.coff;
  f.c = scale * kLog2e;
  f.m[0] = -INFINITY;
  f.l[0] = 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) f.acc[0][db][r] = 0.f;
  f.pos[0] = (r0 + f.l32) % Nq;
  {
    const unsigned short* qrow = q + (qblock + r0 + f.l32) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (f.l32 < nr) raw = *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * f.hl);
      f.qf[0][ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  f.setup_offsets(lane);   // fragment read offsets (its DMA slots are not used)
  // this wave loads whole tiles: LDS-DMA block i covers 16-byte slots
  // 64 i .. 64 i + 63 of the tile
  int koff[kDma], voff[vDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int slot = i * 64 + lane;
    const int r = slot / Cfg<D>::CH, pc = slot % Cfg<D>::CH;
    koff[i] = r * (2 * D) + 16 * (pc ^ Cfg<D>::kswz(r));
  }
#pragma unroll
  for (int i = 0; i < vDma; ++i) {
    const int slot = i * 64 + lane;
    const int r = slot / Cfg<D>::CH, pc = slot % Cfg<D>::CH;
    voff[i] = r * (2 * D) + 16 * (pc ^ Cfg<D>::vswz(r));
  }
  auto load_k = [&](int k0) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc<D>(f.kh, k0, Nk);
#pragma unroll
    for (int i = 0; i < kDma; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(kt + i * 1024), 16, koff[i], 0, 0, 0);
#endif
  };
  auto load_v = [&](int k0) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc<D>(f.vh, k0, Nk);
#pragma unroll
    for (int i = 0; i < vDma; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(vt + i * 1024), 16, voff[i], 0, 0, 0);
#endif
  };

  const int kv_end = CAUSAL ? min(Nk, pmax + 1 + f.coff) : Nk;
  const int n_tiles = (kv_end + kKeys - 1) / kKeys;
  const int n_full = CAUSAL ? min(pmin + f.coff + 1, Nk) / kKeys : Nk / kKeys;

  // One tile: its K and V were queued (K first); refill each slot with the
  // next tile's keys once it has been read.  Loads return in order, so
  // waiting until at most vDma (kDma) loads are outstanding means that the
  // K (V) loads issued before them have landed.
  auto tile = [&](auto mask, auto first, int j) {
    constexpr bool MASK = decltype(mask)::value;
    constexpr bool FIRST = decltype(first)::value;
    const int jn = j + kWaves;
    const bool more = jn < n_tiles;
    f32x16 s[1][F::KB];
    __builtin_amdgcn_s_waitcnt(wait_vm(vDma));
    f.scores(kt, s);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    if (more) load_k(jn * kKeys);
    bf16x8 pf[1][F::PS];
    f.template softmax<MASK, FIRST>(0, s[0], pf[0], j * kKeys);
    if (more) __builtin_amdgcn_s_waitcnt(wait_vm(kDma));
    else      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    f.pv(vt, pf);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    if (more) load_v(jn * kKeys);
  };
  constexpr int kPrefetch = 2;
  unsigned warm[kPrefetch];
  {
    const int64_t lines = ((int64_t)kv_end * 2 * D + 127) / 128;    // per tensor
    const int64_t per = (lines + n_qtiles - 1) / n_qtiles;
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc<D>(f.kh, 0, Nk);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc<D>(f.vh, 0, Nk);
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) {
      const int64_t e = (int64_t)i * kThreads + tid;
      const int64_t line = (int64_t)idx * per + (e % per);
      warm[i] = 0u;
      if (e < 2 * per && line < lines)
        warm[i] = __builtin_amdgcn_raw_buffer_load_b32(e < per ? rk : rv, (int)(line * 128), 0, 0);
    }
  }
  int j = wave;
  if (j < n_tiles) {
    load_k(j * kKeys);
    load_v(j * kKeys);
    if (j >= n_full) tile(std::true_type{}, std::true_type{}, j);
    else             tile(std::false_type{}, std::true_type{}, j);
    j += kWaves;
    for (; j < min(n_full, n_tiles); j += kWaves) tile(std::false_type{}, std::false_type{}, j);
    for (; j < n_tiles; j += kWaves) tile(std::true_type{}, std::false_type{}, j);
  }
  {
    unsigned x = 0u;
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) x ^= warm[i];
    asm volatile("" ::"v"(x));
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
  __syncthreads();

  // Partial results to LDS: the unnormalised O^T of the wave as fp32
  // [32 rows][D] in its K slot (16-byte chunk c of row r at c ^ (r % 16)),
  // its offsets and row sums in its V slot.
  const float l_tot = sum_across_halves(f.l[0]);
  {
    float* ob = reinterpret_cast<float*>(kt);
    float* ml = reinterpret_cast<float*>(vt);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 8 * db + 2 * g + f.hl;    // chunk of dims 32 db + 8 g + 4 hl
        const float4 w = {f.acc[0][db][4 * g], f.acc[0][db][4 * g + 1], f.acc[0][db][4 * g + 2],
                          f.acc[0][db][4 * g + 3]};
        *reinterpret_cast<float4*>(ob + f.l32 * D + 4 * (c ^ (f.l32 & 15))) = w;
      }
    if (f.hl == 0) {
      ml[f.l32] = f.m[0];
      ml[32 + f.l32] = l_tot;
    }
  }
  __syncthreads();

  // Merge: wave w writes head dims [w D/4, (w+1) D/4) of the 32 rows; lane
  // (row, half) takes D/8 of them.  Key 0 is visible to every row and sits
  // in wave 0's first tile, so the row max M is finite; a wave that saw no
  // key of a row (offset -inf) weighs 0.
  const int row = lane & 31, hh = lane >> 5;
  constexpr int NC = D / 32;                   // 16-byte chunks per lane
  float mw[kWaves], M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mw[w] = reinterpret_cast<const float*>(v_lds[w])[row];
    M = fmaxf(M, mw[w]);
  }
  float L = 0.f;
  float out[4 * NC];
#pragma unroll
  for (int e = 0; e < 4 * NC; ++e) out[e] = 0.f;
  const int c0 = wave * (D / 16) + hh * NC;   // first chunk of this lane
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float a = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mw[w] - M) * f.c);
    L += a * reinterpret_cast<const float*>(v_lds[w])[32 + row];
    const float* ob = reinterpret_cast<const float*>(k_lds[w]);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float4 x = *reinterpret_cast<const float4*>(ob + row * D + 4 * ((c0 + c) ^ (row & 15)));
      out[4 * c] += a * x.x;
      out[4 * c + 1] += a * x.y;
      out[4 * c + 2] += a * x.z;
      out[4 * c + 3] += a * x.w;
    }
  }
  if (row >= nr) return;
  const int64_t grow = qblock + r0 + row;
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

// Merge of the key chunks of every row: LSE = log sum_s exp(LSE_s) and
// O = sum_s exp(LSE_s - LSE) O_s, the online-softmax merge applied to whole
// chunks (zzszmyf.github.io notes, sections 5 and 12.1).  One workgroup per
// (row, slice of D/DS head dims), sized so that each lane reads about
// kMergeBatch chunks: a lane reads four head dims of a chunk with one 16-byte
// load (one wave-wide load covers 256 DS/D chunks) and issues kMergeBatch
// such loads before it waits, so a row's chunks arrive in one or two memory
// latencies rather than one after another.  Each lane keeps its own running
// max (the same online rescaling), and the lanes meet at the row max: lane
// groups through shuffles, waves in LDS.  Every slice of a row reads all of
// the row's chunk LSEs, so it has the row max and the denominator itself;
// DS > 1 spreads the few rows of a decoding step over more CUs.  Chunk 0
// always holds key 0, so the row max is finite.
constexpr int kMergeMaxWaves = 16;
constexpr int kMergeBatch = 8;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

// Waves per merge workgroup for `splits` chunks of D/DS dims.
template <int D, int DS>
int merge_waves(int splits) {
  const int64_t lanes = (int64_t)splits * (D / DS / 4);
  return (int)std::max<int64_t>(1, std::min<int64_t>(kMergeMaxWaves, (lanes + 64 * kMergeBatch - 1) / (64 * kMergeBatch)));
}

template <int D, int DS>
__global__ __launch_bounds__(64 * kMergeMaxWaves) void merge_kernel(const float* __restrict__ opart,
                                                                   const float* __restrict__ lpart,
                                                                   unsigned short* __restrict__ o,
                                                                   float* __restrict__ lse,
                                                                   int64_t rows, int splits) {
  constexpr int DW = D / DS;          // head dims of this workgroup
  constexpr int LPS = DW / 4;         // lanes per chunk row, four dims each
  constexpr int SPI = 64 / LPS;       // chunks per wave-wide load
  static_assert(LPS >= 1 && LPS <= 64 && DW % 4 == 0, "merge slice width");
  __shared__ float red[kMergeMaxWaves];
  __shared__ float4 part[kMergeMaxWaves][LPS];
  const int64_t row = blockIdx.x / DS;
  const int dim0 = DW * (int)(blockIdx.x % DS);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nw = blockDim.x >> 6;
  const int step = nw * SPI;          // chunks per pass of the workgroup
  const int sub = lane / LPS, c4 = lane % LPS;

  float m = -INFINITY, sum = 0.f;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int base = wave * SPI + sub; base < splits; base += kMergeBatch * step) {
    // indices past the last chunk read the last one again, with LSE -inf
    float ls[kMergeBatch];
    float4 a[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int64_t sp = min(base + u * step, splits - 1);
      ls[u] = lpart[sp * rows + row];
      a[u] = *reinterpret_cast<const float4*>(opart + (sp * rows + row) * D + dim0 + 4 * c4);
    }
    float mb = m;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      if (base + u * step >= splits) ls[u] = -INFINITY;
      mb = fmaxf(mb, ls[u]);
    }
    const float r = mb == -INFINITY ? 1.f : expf(m - mb);
    sum *= r;
    acc.x *= r;
    acc.y *= r;
    acc.z *= r;
    acc.w *= r;
    m = mb;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float w = ls[u] == -INFINITY ? 0.f : expf(ls[u] - m);
      sum += w;
      acc.x += w * a[u].x;
      acc.y += w * a[u].y;
      acc.z += w * a[u].z;
      acc.w += w * a[u].w;
    }
  }
  // the row max, then every lane's sums relative to it
  float M = wave_max(m);
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = red[0];
  for (int w = 1; w < nw; ++w) M = fmaxf(M, red[w]);
  __syncthreads();
  const float f = m == -INFINITY ? 0.f : expf(m - M);
  sum *= f;
  acc.x *= f;
  acc.y *= f;
  acc.z *= f;
  acc.w *= f;
  // lanes c4, c4 + LPS, ... of a wave hold the same dims of other chunks
#pragma unroll
  for (int off = LPS; off < 64; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off, 64);
    acc.y += __shfl_xor(acc.y, off, 64);
    acc.z += __shfl_xor(acc.z, off, 64);
    acc.w += __shfl_xor(acc.w, off, 64);
    sum += __shfl_xor(sum, off, 64);
  }
  if (sub == 0) part[wave][c4] = acc;
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  if (wave != 0 || lane >= LPS) return;
  float tot = red[0];
  float4 t = part[0][lane];
  for (int w = 1; w < nw; ++w) {
    tot += red[w];
    const float4 p = part[w][lane];
    t.x += p.x;
    t.y += p.y;
    t.z += p.z;
    t.w += p.w;
  }
  const float inv = 1.f / tot;
  const u32x2 out = {pack_bf16x2(t.x * inv, t.y * inv), pack_bf16x2(t.z * inv, t.w * inv)};
  *reinterpret_cast<u32x2*>(o + row * D + dim0 + 4 * lane) = out;
  if (lane == 0 && dim0 == 0) lse[row] = M + logf(tot);
}

// The same merge for many rows: one thread per (row, 8 head dims), each
// walking the chunks itself; enough threads to fill the GPU, where one
// workgroup per row would spend most of its lanes on bookkeeping.
template <int D>
__global__ __launch_bounds__(256) void merge_rows_kernel(const float* __restrict__ opart,
                                                         const float* __restrict__ lpart,
                                                         unsigned short* __restrict__ o,
                                                         float* __restrict__ lse, int64_t rows,
                                                         int splits) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = t / (D / 8);
  const int c8 = (int)(t % (D / 8));
  if (row >= rows) return;
  float mx = -INFINITY;
  for (int sp = 0; sp < splits; ++sp) mx = fmaxf(mx, lpart[(int64_t)sp * rows + row]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float sum = 0.f;
  for (int sp = 0; sp < splits; ++sp) {
    const float ls = lpart[(int64_t)sp * rows + row];
    const float w = ls == -INFINITY ? 0.f : expf(ls - mx);
    sum += w;
    const float4* src = reinterpret_cast<const float4*>(opart + ((int64_t)sp * rows + row) * D + 8 * c8);
    const float4 a = src[0], b = src[1];
    acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
    acc[4] += w * b.x; acc[5] += w * b.y; acc[6] += w * b.z; acc[7] += w * b.w;
  }
  const float inv = 1.f / sum;
  const u32x4 out = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                     pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  *reinterpret_cast<u32x4*>(o + row * D + 8 * c8) = out;
  if (c8 == 0) lse[row] = mx + logf(sum);
}

// Rows above which the merge runs one thread per (row, 8 dims).
constexpr int64_t kMergeRowsMin = 4096;
// Below it, a row's head dims are split over up to D/16 workgroups until the
// merge has at least this many.
constexpr int64_t kMergeMinGrid = 256;

template <int D, int DS>
void launch_merge(const float* opart, const float* lpart, unsigned short* o, float* lse, int64_t rows,
                  int splits, hipStream_t stream) {
  hipLaunchKernelGGL((merge_kernel<D, DS>), dim3((unsigned)(rows * DS)), dim3(64 * merge_waves<D, DS>(splits)), 0,
                     stream, opart, lpart, o, lse, rows, splits);
}
// Up to this many 128-row workgroups (three quarters of the 256 CUs) a call
// with at least kWsMinTiles key tiles runs fwd_bf16_ws_kernel instead:
// 32-row workgroups whose four waves split the keys.  Measured against the
// 128-row kernel: faster at 128 and 192 workgroups (d = 64 and 128, causal
// or not), slower at 240 and 256 (d = 128 non-causal at 256: 62 vs 40 us).
constexpr int64_t kWsMaxGrid = 192;
constexpr int kWsMinTiles = 8;
// Workgroups from which d = 64 takes 256-row tiles: two per CU of the 256.
constexpr int64_t kWideTileMinGrid = 512;

template <int D, bool CAUSAL>
hipError_t launch(const GqaProblem& p, hipStream_t stream) {
  constexpr int BR = 32 * kWaves;
  static_assert(BR == kTileRows, "host tiling and kernel tile height differ");
  const QueryTiling t = query_tiling(p.H / p.Hkv, p.Nq, p.causal);
  const int BHkv = p.B * p.Hkv;
  const int G = p.H / p.Hkv;
  const dim3 block(kThreads);
  const unsigned short* q = static_cast<const unsigned short*>(p.q);
  const unsigned short* k = static_cast<const unsigned short*>(p.k);
  const unsigned short* v = static_cast<const unsigned short*>(p.v);
  // d = 64 leaves half the registers free at 32 rows per wave: 64 rows per
  // wave (two 32-row blocks sharing every K and V fragment read) halve the
  // LDS reads and the L2-to-LDS bytes per product, and still fit two
  // workgroups per CU.  Taken when the 256-row tiles give at least two
  // workgroups per CU of the 256.
  if constexpr (D == 64) {
    if (p.splits == 1) {
      const QueryTiling t2 = query_tiling(G, p.Nq, p.causal, 2 * BR);
      if (t2.n_qtiles * BHkv >= kWideTileMinGrid) {
        const dim3 grid((unsigned)(t2.n_qtiles * BHkv));
        hipLaunchKernelGGL((fwd_bf16_kernel<D, 2, CAUSAL, false>), grid, block, 0, stream, q, k, v,
                           static_cast<unsigned short*>(p.o), p.lse, p.Nq, p.Nk, G, BHkv,
                           (int)t2.n_qtiles, t2.tph, p.scale, 1, nullptr, nullptr,
                           xcd_head_group(BHkv, t2.n_qtiles, G, t2.tph, 1));
        return hipGetLastError();
      }
    }
  }
  if (p.splits == 1 && t.n_qtiles * BHkv <= kWsMaxGrid && (p.Nk + kKeys - 1) / kKeys >= kWsMinTiles) {
    const QueryTiling t32 = query_tiling(G, p.Nq, p.causal, 32);
    const dim3 grid((unsigned)(t32.n_qtiles * BHkv));
    hipLaunchKernelGGL((fwd_bf16_ws_kernel<D, CAUSAL>), grid, block, 0, stream, q, k, v,
                       static_cast<unsigned short*>(p.o), p.lse, p.Nq, p.Nk, G, BHkv, (int)t32.n_qtiles,
                       t32.tph, p.scale, xcd_head_group(BHkv, t32.n_qtiles, G, t32.tph, 1));
    return hipGetLastError();
  }
  if (p.splits == 1) {
    const dim3 grid((unsigned)(t.n_qtiles * BHkv));
    hipLaunchKernelGGL((fwd_bf16_kernel<D, 1, CAUSAL, false>), grid, block, 0, stream, q, k, v,
                       static_cast<unsigned short*>(p.o), p.lse, p.Nq, p.Nk, G, BHkv,
                       (int)t.n_qtiles, t.tph, p.scale, 1, nullptr, nullptr,
                       xcd_head_group(BHkv, t.n_qtiles, G, t.tph, 1));
    return hipGetLastError();
  }
  const SplitLayout L = splitkv_layout(p.B, p.H, p.Nq, p.d, p.splits);
  float* opart = static_cast<float*>(p.workspace);
  float* lpart = reinterpret_cast<float*>(static_cast<unsigned char*>(p.workspace) + L.lse_offset);
  const dim3 grid((unsigned)(t.n_qtiles * p.splits * BHkv));
  hipLaunchKernelGGL((fwd_bf16_kernel<D, 1, CAUSAL, true>), grid, block, 0, stream, q, k, v,
                     nullptr, nullptr, p.Nq, p.Nk, G, BHkv, (int)t.n_qtiles, t.tph, p.scale,
                     p.splits, opart, lpart, xcd_head_group(BHkv, t.n_qtiles, G, t.tph, p.splits));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)p.B * p.H * p.Nq;
  if (rows >= kMergeRowsMin) {
    const int64_t threads = rows * (D / 8);
    hipLaunchKernelGGL((merge_rows_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, opart, lpart, static_cast<unsigned short*>(p.o), p.lse, rows, p.splits);
  } else {
    unsigned short* o = static_cast<unsigned short*>(p.o);
    if (rows * 4 < kMergeMinGrid && D >= 128) launch_merge<D, D / 16>(opart, lpart, o, p.lse, rows, p.splits, stream);
    else if (rows * 2 < kMergeMinGrid) launch_merge<D, 4>(opart, lpart, o, p.lse, rows, p.splits, stream);
    else if (rows < kMergeMinGrid) launch_merge<D, 2>(opart, lpart, o, p.lse, rows, p.splits, stream);
    else launch_merge<D, 1>(opart, lpart, o, p.lse, rows, p.splits, stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const GqaProblem& p, hipStream_t stream) {
  if (p.d == 64) return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace fa
