// Internal declarations shared by the host entry points and the kernels'
// launch wrappers.  Not part of the public interface (that is fa_fwd.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Problem description handed from the validated entry point to a launcher.
struct Problem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d;
  float scale;
  int causal;
};

// bf16 problem: B*H query heads of Nq rows over B*Hkv K/V heads of Nk keys
// (query head h reads K/V head h / (H / Hkv)); with splits > 1 the keys of
// every query tile are cut into `splits` chunks whose partial results go to
// `workspace` (layout in splitkv_layout) before a merge writes o and lse.
struct GqaProblem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  int splits;
  void* workspace;
};

// Backward problem (bf16, Nq = Nk = N): gradients dq, dk, dv of O =
// softmax(scale Q K^T) V for the upstream gradient dout, from the forward's
// o and lse.  q, o, dout, dq are [B,H,N,d]; k, v, dk, dv are [B,Hkv,N,d],
// query head h reading K/V head h / (H/Hkv).  `workspace` holds the per-row
// D = <dO, O> (fp32 [B*H*N]) and, when Hkv < H, the per-query-head fp32
// partial dK and dV ([B*H, N, d] each) that are summed over each group.
struct BwdProblem {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int B, H, Hkv, N, d;
  float scale;
  int causal;
  void* workspace;
};

struct BwdLayout {
  int64_t d_bytes, dk_offset, dv_offset, total;
};
inline BwdLayout bwd_layout(int B, int H, int Hkv, int N, int d) {
  BwdLayout L;
  L.d_bytes = ((int64_t)B * H * N * 4 + 255) / 256 * 256;
  const int64_t part = Hkv < H ? ((int64_t)B * H * N * d * 4 + 255) / 256 * 256 : 0;
  L.dk_offset = L.d_bytes;
  L.dv_offset = L.d_bytes + part;
  L.total = L.d_bytes + 2 * part;
  return L;
}
inline int64_t bwd_workspace_bytes(int B, int H, int N) { return bwd_layout(B, H, H, N, 64).total; }

// fp8 problem (square): MX-quantized Q, K (codes [B*H*N, d], E8M0 scales
// [B*H*N, d/32]) and V (transposed 64-key tiles and their scales, as written
// by the V quantizer); o bf16 [B,H,N,d], lse fp32 [B,H,N].
struct Fp8Problem {
  const void* q8;
  const void* qs;
  const void* k8;
  const void* ks;
  const void* v8t;
  const void* vs;
  void* o;
  float* lse;
  int B, H, Hkv, N, d;   // K and V of B*Hkv heads; query head h reads K/V head h / (H/Hkv)
  float scale;
  int causal;
};

// Bytes of the quantized V of B*H heads: codes and scales.
inline int64_t fp8_v_code_bytes(int64_t BH, int N, int d) { return BH * ((N + 63) / 64) * d * 64; }
inline int64_t fp8_v_scale_bytes(int64_t BH, int N, int d) { return BH * ((N + 63) / 64) * 2 * d; }

// Query rows per workgroup tile of the bf16 kernel.
constexpr int kTileRows = 128;

// Heads an XCD runs at a time in the block order of xcd_order (0, heads
// varying fastest, when BH, the number of K/V heads over the batch, is not a
// multiple of 8, or when a head has a single query tile, so that no two
// blocks read the same keys).  One at a time reads the least from memory, but
// a group's last blocks start late, so its heaviest block must stay short
// next to the time a group takes.  Causal query tiles (tph > 0 per query
// head, G query heads per K/V head) weigh 1..tph, so the heaviest of `splits`
// key chunks is tph/splits of a head's G*tph^2/2; an XCD holds 64 workgroups
// at once (32 CUs, two each).  The group is sized so the heaviest block takes
// at most a group's time per slot (G*tph^2/2 * hg / 64): a list-scheduling
// simulation of the dispatch and the measured times agree that the makespan
// then stays at its ideal (C4 runs one head at a time per XCD at the same
// speed as two, with a third of the memory traffic; C3, four heads at a
// time, is 3 % faster than with all eight).
// `spread` scales that bound: the fp8 kernel, which is not held by the power
// limit and so is bound by cycles rather than by data movement, keeps the
// heaviest block to half a group's time (spread 4; C4 fp8 3 % faster than at
// spread 2).
inline int xcd_head_group(int64_t BH, int64_t qtiles, int G, int tph, int splits, int spread = 2) {
  if (BH % 8 != 0 || qtiles <= 1) return 0;
  const int hx = (int)(BH / 8);   // heads per XCD
  if (tph == 0) return 1;         // equal tiles
  constexpr int64_t kXcdSlots = 64;
  const int64_t den = (int64_t)splits * G * tph;
  const int64_t need = (spread * kXcdSlots + den - 1) / den;
  int g = need >= hx ? hx : (int)need;
  while (hx % g != 0) ++g;
  return g;
}

// How the G*Nq query rows that share one K/V head are cut into tiles.
// tph > 0: tph tiles per query head, never crossing heads (long causal heads:
// tiles can be ordered heaviest first); tph == 0: tiles packed across the G
// heads (all other cases; a decoding step of G heads then reads K/V once).
struct QueryTiling {
  int tph;
  int64_t n_qtiles;   // tiles per K/V head
};
inline QueryTiling query_tiling(int G, int Nq, int causal, int rows = kTileRows) {
  QueryTiling t;
  if (causal && Nq >= rows) {
    t.tph = (Nq + rows - 1) / rows;
    t.n_qtiles = (int64_t)G * t.tph;
  } else {
    t.tph = 0;
    t.n_qtiles = ((int64_t)G * Nq + rows - 1) / rows;
  }
  return t;
}

// Workspace layout of the key-split path: partial outputs, fp32
// [splits][B*H*Nq][d], then partial LSEs, fp32 [splits][B*H*Nq], each part
// starting on a 256-byte boundary.
struct SplitLayout {
  int64_t o_bytes, lse_offset, total;
};
inline SplitLayout splitkv_layout(int B, int H, int Nq, int d, int splits) {
  const int64_t rows = (int64_t)B * H * Nq;
  SplitLayout L;
  L.o_bytes = (int64_t)splits * rows * d * 4;
  L.lse_offset = (L.o_bytes + 255) / 256 * 256;
  L.total = L.lse_offset + ((int64_t)splits * rows * 4 + 255) / 256 * 256;
  return L;
}

// Bytes of the static device scratch that the allocation-free key-split call
// uses in place of a caller's workspace (one copy per GPU).
constexpr int64_t kNoAllocScratchBytes = int64_t(32) << 20;

// Device address of that scratch on the GPU `stream` belongs to; looked up
// once per GPU and cached.  Returns the HIP status of the lookup.
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);

// Each launcher queues its kernels on `stream` and returns the HIP status of
// the launch (hipSuccess or the runtime's error).
hipError_t launch_fwd_f32(const Problem& p, hipStream_t stream);
hipError_t launch_fwd_bf16(const GqaProblem& p, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdProblem& p, hipStream_t stream);
hipError_t launch_quantize_qk_fp8(const void* x, int64_t rows, int d, void* x8, void* xs, hipStream_t stream);
hipError_t launch_quantize_qk_fp8_rotated(const void* x, int64_t rows, int d, const void* signs, void* x8,
                                          void* xs, hipStream_t stream);
hipError_t launch_quantize_v_fp8(const void* v, int BH, int N, int d, void* v8t, void* vs, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8Problem& p, hipStream_t stream);

}  // namespace fa
