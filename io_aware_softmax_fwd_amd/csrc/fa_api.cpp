// C entry points of libfa_fwd.so (declared in include/fa_fwd.h).
//
// Every argument is checked on the host before any HIP call, so a bad call
// returns its status without touching the device (and can be tested on a
// machine with no GPU).  Valid calls are forwarded to the kernel launchers.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <initializer_list>
#include <utility>

#include "fa_fwd.h"
#include "fa_internal.h"

namespace {

// Largest supported problem: element offsets stay far inside int64.
constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int kMaxSplits = 256;
// A dispatch carries its size in 32-bit work-item counts, so every launch
// must stay below 2^32 threads: 2^24 workgroups of 256 threads.
constexpr int64_t kMaxWorkgroups = int64_t(1) << 24;

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Workgroup count bound of the square problems: no launch takes more than
// one 256-thread workgroup per 32 query rows (or keys) of a head.
bool grid_too_large(int64_t heads, int64_t rows_per_head) {
  return heads * ((rows_per_head + 31) / 32) >= kMaxWorkgroups;
}

bool overlap(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)b_bytes && b0 < a0 + (uintptr_t)a_bytes;
}

int validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
             int B, int H, int N, int d, float scale, int causal, int elem_bytes) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_D;
  const int64_t rows = (int64_t)B * H * N;
  if (rows * d >= kMaxElems || grid_too_large((int64_t)B * H, N)) return FA_ERR_SHAPE;
  // One head's K or V (N x d) must stay below 2 GiB: the kernels address a
  // head with 32-bit byte offsets.
  if ((int64_t)N * d * elem_bytes >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (causal != 0 && causal != 1) return FA_ERR_CAUSAL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
    return FA_ERR_ALIGN;
  const int64_t tb = rows * d * elem_bytes, lb = rows * 4;
  if (overlap(o, tb, q, tb) || overlap(o, tb, k, tb) || overlap(o, tb, v, tb) ||
      overlap(lse, lb, q, tb) || overlap(lse, lb, k, tb) || overlap(lse, lb, v, tb) ||
      overlap(lse, lb, o, tb))
    return FA_ERR_ALIAS;
  return FA_OK;
}

// Checks of the general bf16 call (grouped K/V heads, Nq != Nk, key
// splits).  A workspace is required only when splits > 1 and need_ws is set
// (the allocation-free call brings its own).
int validate_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int splits,
                 const void* ws, size_t ws_bytes, bool need_ws = true) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Hkv < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (H % Hkv != 0) return FA_ERR_HEADS;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_D;
  const int64_t qrows = (int64_t)B * H * Nq, krows = (int64_t)B * Hkv * Nk;
  if (qrows * d >= kMaxElems || krows * d >= kMaxElems) return FA_ERR_SHAPE;
  // One K/V head below 2 GiB (32-bit byte offsets inside a head) and the
  // query rows of one K/V head below 2^31.
  if ((int64_t)Nk * d * 2 >= (int64_t(1) << 31) || (int64_t)Nq * d * 2 >= (int64_t(1) << 31) ||
      (int64_t)(H / Hkv) * Nq >= (int64_t(1) << 31))
    return FA_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (causal != 0 && causal != 1) return FA_ERR_CAUSAL;
  if (causal && Nq > Nk) return FA_ERR_SHAPE;
  if (splits < 1 || splits > kMaxSplits) return FA_ERR_SPLITS;
  const fa::QueryTiling t = fa::query_tiling(H / Hkv, Nq, causal);
  // every launch of the call: at most this many 256-thread workgroups
  // (the 32-row kernel for small grids runs only when the 128-row grid is
  // under 192 workgroups)
  if (t.n_qtiles * splits * B * Hkv >= kMaxWorkgroups) return FA_ERR_SHAPE;
  // the merge's 1-D grid: one thread per (query row, 8 head dims)
  if (splits > 1 && qrows * (d / 8) >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
    return FA_ERR_ALIGN;
  const int64_t qb = qrows * d * 2, kb = krows * d * 2, lb = qrows * 4;
  if (overlap(o, qb, q, qb) || overlap(o, qb, k, kb) || overlap(o, qb, v, kb) ||
      overlap(lse, lb, q, qb) || overlap(lse, lb, k, kb) || overlap(lse, lb, v, kb) ||
      overlap(lse, lb, o, qb))
    return FA_ERR_ALIAS;
  if (splits > 1 && need_ws) {
    const fa::SplitLayout L = fa::splitkv_layout(B, H, Nq, d, splits);
    if (!ws || (int64_t)ws_bytes < L.total) return FA_ERR_WORKSPACE;
    if (misaligned(ws)) return FA_ERR_ALIGN;
    if (overlap(ws, L.total, q, qb) || overlap(ws, L.total, k, kb) || overlap(ws, L.total, v, kb) ||
        overlap(ws, L.total, o, qb) || overlap(ws, L.total, lse, lb))
      return FA_ERR_ALIAS;
  }
  return FA_OK;
}

// Chunks per row block, from the workgroups one chunk level gives (base) and
// the 64-key tiles of a row (tiles).  Measured on decoding with 1 to 32 K/V
// heads over 4K to 128K keys: a chunk streams best at 16 or more tiles, the
// GPU fills at two workgroups per CU, and a merge over hundreds of chunks per
// row costs more than it saves.  So: two workgroups per CU when chunks keep
// 16 tiles (doubling up to four per CU while they still do); else, when that
// takes at most 128 chunks, two per CU with chunks of at least 4 tiles;
// else one per CU, with chunks of 8 tiles if the keys allow, else of 4.
int choose_splits(int B, int H, int Hkv, int Nq, int Nk, int causal, int num_cus) {
  if (B < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 || Nq < 1 || Nk < 1) return 1;
  if (num_cus < 1) num_cus = 256;
  const int64_t base = fa::query_tiling(H / Hkv, Nq, causal != 0).n_qtiles * B * Hkv;
  const int64_t tiles = (Nk + 63) / 64;
  const int64_t s1 = (num_cus + base - 1) / base;
  const int64_t s2 = (2 * (int64_t)num_cus + base - 1) / base;
  const int64_t s4 = (4 * (int64_t)num_cus + base - 1) / base;
  int64_t s;
  if (tiles >= 16 * s2) {
    s = s2;
    while (2 * s <= s4 && tiles >= 16 * 2 * s) s *= 2;
  } else if (s2 <= 128) {
    s = std::min<int64_t>(s2, tiles / 4);
  } else if (tiles >= 8 * s1) {
    s = s1;
  } else {
    s = std::min<int64_t>(s1, tiles / 4);
  }
  return (int)std::max<int64_t>(1, std::min<int64_t>(s, kMaxSplits));
}

int validate_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, const void* dq, const void* dk, const void* dv, int B, int H,
                 int Hkv, int N, int d, float scale, int causal, const void* ws, size_t ws_bytes) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Hkv < 1 || N < 1) return FA_ERR_SHAPE;
  if (H % Hkv != 0) return FA_ERR_HEADS;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_D;
  const int64_t rows = (int64_t)B * H * N;
  if (rows * d >= kMaxElems || grid_too_large((int64_t)B * H, N)) return FA_ERR_SHAPE;
  if ((int64_t)N * d * 2 >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (causal != 0 && causal != 1) return FA_ERR_CAUSAL;
  const void* all[] = {q, k, v, o, dout, lse, dq, dk, dv, ws};
  for (const void* p : all)
    if (p && misaligned(p)) return FA_ERR_ALIGN;
  const int64_t wb = fa::bwd_layout(B, H, Hkv, N, d).total;
  if (!ws || (int64_t)ws_bytes < wb) return FA_ERR_WORKSPACE;
  // outputs (dq, dk, dv, workspace) overlap nothing else
  const int64_t tb = rows * d * 2, kb = (int64_t)B * Hkv * N * d * 2, lb = rows * 4;
  const void* ptr[] = {q, k, v, o, dout, lse, dq, dk, dv, ws};
  const int64_t len[] = {tb, kb, kb, tb, tb, lb, tb, kb, kb, wb};
  for (int a = 6; a < 10; ++a)
    for (int b = 0; b < 10; ++b)
      if (a != b && overlap(ptr[a], len[a], ptr[b], len[b])) return FA_ERR_ALIAS;
  return FA_OK;
}

bool any_misaligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (misaligned(p)) return true;
  return false;
}

bool any_overlap(const void* out, int64_t out_bytes, std::initializer_list<std::pair<const void*, int64_t>> ins) {
  for (const auto& in : ins)
    if (overlap(out, out_bytes, in.first, in.second)) return true;
  return false;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int causal, hipStream_t stream) {
  const int st = validate(q, k, v, o, lse, B, H, N, d, scale, causal, 2);
  if (st != FA_OK) return st;
  const fa::GqaProblem p{q, k, v, o, lse, B, H, H, N, N, d, scale, causal, 1, nullptr};
  return fa::launch_fwd_bf16(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, hipStream_t stream) {
  const int st = validate(q, k, v, o, lse, B, H, N, d, scale, causal, 4);
  if (st != FA_OK) return st;
  const fa::Problem p{q, k, v, o, lse, B, H, N, d, scale, causal};
  return fa::launch_fwd_f32(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_fwd_splitkv_workspace_size(int B, int H, int Nq, int d, int num_splits) {
  if (B < 1 || H < 1 || Nq < 1 || (d != 64 && d != 128) || num_splits < 1 || num_splits > kMaxSplits)
    return 0;
  return (size_t)fa::splitkv_layout(B, H, Nq, d, num_splits).total;
}

int fa_fwd_splitkv_num_splits(int B, int H, int Nq, int Nk, int num_cus) {
  // causal and non-causal calls cut a head's queries into the same tiles
  // when every K/V head serves one query head
  return choose_splits(B, H, H, Nq, Nk, 0, num_cus);
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int Nq, int Nk, int d, float scale, int causal, int num_splits, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  const int st = validate_gqa(q, k, v, o, lse, B, H, H, Nq, Nk, d, scale, causal, num_splits,
                              workspace, workspace_bytes);
  if (st != FA_OK) return st;
  // the workspace is part of this entry point's contract even for one split
  if (!workspace || workspace_bytes < fa_fwd_splitkv_workspace_size(B, H, Nq, d, num_splits))
    return FA_ERR_WORKSPACE;
  if (misaligned(workspace)) return FA_ERR_ALIGN;
  const fa::GqaProblem p{q, k, v, o, lse, B, H, H, Nq, Nk, d, scale, causal, num_splits, workspace};
  return fa::launch_fwd_bf16(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_fwd_splitkv_noalloc_max_bytes(void) { return (size_t)fa::kNoAllocScratchBytes; }

int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int Nq, int Nk, int d, float scale, int causal, int num_splits,
                           hipStream_t stream) {
  const int st = validate_gqa(q, k, v, o, lse, B, H, H, Nq, Nk, d, scale, causal, num_splits,
                              nullptr, 0, false);
  if (st != FA_OK) return st;
  if (fa::splitkv_layout(B, H, Nq, d, num_splits).total > fa::kNoAllocScratchBytes) return FA_ERR_SCRATCH;
  void* scratch = nullptr;
  if (fa::noalloc_scratch(stream, &scratch) != hipSuccess) return FA_ERR_HIP;
  const fa::GqaProblem p{q, k, v, o, lse, B, H, H, Nq, Nk, d, scale, causal, num_splits, scratch};
  return fa::launch_fwd_bf16(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_gqa_num_splits(int B, int H, int Hkv, int Nq, int Nk, int causal, int num_cus) {
  return choose_splits(B, H, Hkv, Nq, Nk, causal, num_cus);
}

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int Hkv, int Nq, int Nk, int d, float scale, int causal, int num_splits,
               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = validate_gqa(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, num_splits,
                              workspace, workspace_bytes);
  if (st != FA_OK) return st;
  const fa::GqaProblem p{q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, num_splits,
                         num_splits > 1 ? workspace : nullptr};
  return fa::launch_fwd_bf16(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  return (size_t)fa::bwd_layout(B, H, H, N, d).total;
}

size_t fa_bwd_gqa_workspace_size(int B, int H, int Hkv, int N, int d) {
  if (B < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 || N < 1 || (d != 64 && d != 128)) return 0;
  if ((int64_t)B * H * N * d >= kMaxElems) return 0;
  return (size_t)fa::bwd_layout(B, H, Hkv, N, d).total;
}

int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
               float scale, int causal, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = validate_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal,
                              workspace, workspace_bytes);
  if (st != FA_OK) return st;
  const fa::BwdProblem p{q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, workspace};
  return fa::launch_bwd_bf16(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
           int causal, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, scale, causal, workspace,
                    workspace_bytes, stream);
}

int fa_quantize_qk_fp8(const void* x, int64_t rows, int d, void* x8, void* xs, hipStream_t stream) {
  if (!x || !x8 || !xs) return FA_ERR_NULL;
  if (rows < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_D;
  // one thread per 32-element block: below 2^32 threads
  if (rows * d >= kMaxElems || rows * (d / 32) >= kMaxWorkgroups * 256) return FA_ERR_SHAPE;
  if (any_misaligned({x, x8, xs})) return FA_ERR_ALIGN;
  const int64_t xb = rows * d * 2, cb = rows * d, sb = rows * (d / 32);
  if (any_overlap(x8, cb, {{x, xb}, {xs, sb}}) || any_overlap(xs, sb, {{x, xb}})) return FA_ERR_ALIAS;
  return fa::launch_quantize_qk_fp8(x, rows, d, x8, xs, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_quantize_qk_fp8_rotated(const void* x, int64_t rows, int d, const signed char* signs, void* x8,
                               void* xs, hipStream_t stream) {
  if (!x || !x8 || !xs) return FA_ERR_NULL;
  if (rows < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_D;
  // one thread per 32-element block: below 2^32 threads
  if (rows * d >= kMaxElems || rows * (d / 32) >= kMaxWorkgroups * 256) return FA_ERR_SHAPE;
  if (any_misaligned({x, x8, xs})) return FA_ERR_ALIGN;
  const int64_t xb = rows * d * 2, cb = rows * d, sb = rows * (d / 32);
  if (any_overlap(x8, cb, {{x, xb}, {xs, sb}}) || any_overlap(xs, sb, {{x, xb}})) return FA_ERR_ALIAS;
  if (signs && (any_overlap(x8, cb, {{signs, d}}) || any_overlap(xs, sb, {{signs, d}}))) return FA_ERR_ALIAS;
  return fa::launch_quantize_qk_fp8_rotated(x, rows, d, signs, x8, xs, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_fp8_v_bytes(int BH, int N, int d) {
  if (BH < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  return (size_t)fa::fp8_v_code_bytes(BH, N, d);
}

size_t fa_fp8_v_scale_bytes(int BH, int N, int d) {
  if (BH < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  return (size_t)fa::fp8_v_scale_bytes(BH, N, d);
}

int fa_quantize_v_fp8(const void* v, int BH, int N, int d, void* v8t, void* vs, hipStream_t stream) {
  if (!v || !v8t || !vs) return FA_ERR_NULL;
  if (BH < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_D;
  if ((int64_t)BH * N * d >= kMaxElems || (int64_t)N * d * 2 >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  // 2d threads per 64-key block: below 2^32 threads
  if ((int64_t)BH * ((N + 63) / 64) * 2 * d >= kMaxWorkgroups * 256) return FA_ERR_SHAPE;
  if (any_misaligned({v, v8t, vs})) return FA_ERR_ALIGN;
  const int64_t vb = (int64_t)BH * N * d * 2, cb = fa::fp8_v_code_bytes(BH, N, d),
                sb = fa::fp8_v_scale_bytes(BH, N, d);
  if (any_overlap(v8t, cb, {{v, vb}, {vs, sb}}) || any_overlap(vs, sb, {{v, vb}})) return FA_ERR_ALIAS;
  return fa::launch_quantize_v_fp8(v, BH, N, d, v8t, vs, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_fp8_gqa(const void* q8, const void* qs, const void* k8, const void* ks, const void* v8t,
                   const void* vs, void* o, float* lse, int B, int H, int Hkv, int N, int d, float scale,
                   int causal, hipStream_t stream) {
  if (!q8 || !qs || !k8 || !ks || !v8t || !vs || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Hkv < 1 || N < 1) return FA_ERR_SHAPE;
  if (H % Hkv != 0) return FA_ERR_HEADS;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_D;
  const int64_t rows = (int64_t)B * H * N;
  if (rows * d >= kMaxElems || (int64_t)N * d * 2 >= (int64_t(1) << 31) || grid_too_large((int64_t)B * H, N))
    return FA_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (causal != 0 && causal != 1) return FA_ERR_CAUSAL;
  if (any_misaligned({q8, qs, k8, ks, v8t, vs, o, lse})) return FA_ERR_ALIGN;
  const int64_t kvrows = (int64_t)B * Hkv * N;
  const int64_t cb = rows * d, sb = rows * (d / 32), kcb = kvrows * d, ksb = kvrows * (d / 32),
                ob = rows * d * 2, lb = rows * 4, vcb = fa::fp8_v_code_bytes((int64_t)B * Hkv, N, d),
                vsb = fa::fp8_v_scale_bytes((int64_t)B * Hkv, N, d);
  const std::initializer_list<std::pair<const void*, int64_t>> ins = {
      {q8, cb}, {qs, sb}, {k8, kcb}, {ks, ksb}, {v8t, vcb}, {vs, vsb}};
  if (any_overlap(o, ob, ins) || any_overlap(lse, lb, ins) || overlap(o, ob, lse, lb)) return FA_ERR_ALIAS;
  const fa::Fp8Problem p{q8, qs, k8, ks, v8t, vs, o, lse, B, H, Hkv, N, d, scale, causal};
  return fa::launch_fwd_fp8(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_fp8(const void* q8, const void* qs, const void* k8, const void* ks, const void* v8t, const void* vs,
               void* o, float* lse, int B, int H, int N, int d, float scale, int causal, hipStream_t stream) {
  return fa_fwd_fp8_gqa(q8, qs, k8, ks, v8t, vs, o, lse, B, H, H, N, d, scale, causal, stream);
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H, N must be >= 1, B*H*N*d below 2^40, B*H*ceil(N/32) below 2^24 and one head below 2 GiB";
    case FA_ERR_UNSUPPORTED_D: return "head dimension must be 64 or 128";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_ALIGN: return "pointers must be 16-byte aligned";
    case FA_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    case FA_ERR_CAUSAL: return "causal must be 0 or 1";
    case FA_ERR_ALIAS: return "an output or the workspace overlaps another buffer";
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than the size query returns";
    case FA_ERR_SPLITS: return "num_splits must be between 1 and 256";
    case FA_ERR_HEADS: return "H must be a multiple of Hkv";
    case FA_ERR_SCRATCH: return "the key-split partials exceed the static scratch (fa_fwd_splitkv_noalloc_max_bytes); use fa_fwd_splitkv with a workspace";
    default: return "unknown status";
  }
}

}  // extern "C"
