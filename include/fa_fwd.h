/*
 * fa_fwd.h -- fused exact-attention forward pass for AMD MI355X (gfx950).
 *
 * Computes, for every batch b, head h and query row i,
 *
 *     O[b,h,i,:]  = sum_j softmax_j(scale * <q_i, k_j>) * v_j
 *     LSE[b,h,i]  = log( sum_j exp(scale * <q_i, k_j>) )          (natural log)
 *
 * with j over all keys, or over j <= i when `causal` is 1.  The problem is the
 * one stated by the zzszmyf.github.io notes "FlashAttention 原理是什么？为什么又省
 * 显存又快": Q, K, V of N x d per head in device memory, exact
 * softmax(Q K^T) V returned with O(N) extra memory (section 7.2, Theorem 1),
 * with the per-row softmax statistics kept for a recomputing backward pass
 * (section 6), here folded into one log-sum-exp per row.  The N x N score and
 * probability matrices never reach device memory: K/V are streamed tile by
 * tile and merged with a running row max and row sum (aiqz.cc Flash
 * Attention IO article, section 在线Softmax算法).
 *
 * Layout: every tensor is dense row-major [B, H, N, d] (d fastest); LSE is
 * [B, H, N] float32.  O has the input element type.
 *
 * Ownership: the caller allocates and owns every buffer.  The library
 * allocates nothing, keeps no state between calls and is thread-safe.  O and
 * LSE must not overlap Q, K, V or each other.
 *
 * Errors: argument errors are detected on the host before any HIP call and
 * returned synchronously (no work is queued).  A failed kernel launch returns
 * FA_ERR_HIP.  The work itself runs asynchronously on `stream` (0 = the null
 * stream); a fault during execution surfaces at the caller's next
 * synchronisation of that stream.
 */
#ifndef FA_FWD_H
#define FA_FWD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,           /* a required pointer is NULL                     */
  FA_ERR_SHAPE = 2,          /* B, H or N < 1, or the problem is too large     */
  FA_ERR_UNSUPPORTED_D = 3,  /* head dimension other than 64 or 128            */
  FA_ERR_SCALE = 4,          /* scale not finite or not > 0                    */
  FA_ERR_ALIGN = 5,          /* a pointer is not 16-byte aligned               */
  FA_ERR_HIP = 6,            /* the HIP runtime refused the launch             */
  FA_ERR_CAUSAL = 7,         /* causal flag other than 0 or 1                  */
  FA_ERR_ALIAS = 8,          /* an output or the workspace overlaps a buffer   */
  FA_ERR_WORKSPACE = 9,      /* workspace NULL or smaller than required        */
  FA_ERR_SPLITS = 10,        /* num_splits outside 1..256                      */
  FA_ERR_HEADS = 11,         /* H is not a multiple of Hkv                     */
  FA_ERR_SCRATCH = 12        /* key-split partials exceed the static scratch   */
};

/*
 * bfloat16 attention forward: the hot path.
 *   q, k, v : device pointers, [B,H,N,d] bfloat16 (raw 16-bit storage).
 *   o       : device pointer, [B,H,N,d] bfloat16, written (round to nearest
 *             even from the fp32 result).
 *   lse     : device pointer, [B,H,N] float32, written.
 *   B, H, N : batch, heads, sequence length (N >= 1; any N, no tile multiple
 *             needed).  B*H*N*d must stay below 2^40 elements,
 *             B*H*ceil(N/32) below 2^24 (no launch may exceed 2^32
 *             threads, the dispatch limit; 256 threads serve at most 32
 *             rows) and one head (N*d elements) below 2 GiB.
 *   d       : head dimension, 64 or 128.
 *   scale   : multiplier of Q K^T before the softmax, finite and > 0
 *             (usually 1/sqrt(d)).
 *   causal  : 1 -> key j attends to query i only when j <= i; 0 -> all keys.
 *   stream  : HIP stream the kernel is queued on.
 * Products are taken on bf16 matrix cores with fp32 accumulation; the
 * softmax statistics, the rescaling and the final division are fp32.
 * Range of V: the exponent offset may lag the running row max, so a tile's
 * unnormalised probabilities can reach 2^48 before the offset moves, and
 * the fp32 output accumulators can reach about 2^79 * max|v| (fewer than
 * 2^31 keys).  O is finite and within the stated accuracy for
 * max|v| < 2^48 (about 2.8e14); beyond that the accumulators may overflow
 * to inf or NaN where the exact result is finite.  Q and K have no such
 * limit (the scores themselves are exact fp32 products of bf16 values).
 * Returns an fa_status.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal,
           hipStream_t stream);

/*
 * float32 twin of fa_fwd: q, k, v, o are [B,H,N,d] float32 and every
 * product, sum and exponential is fp32.  Same argument rules and errors.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o,
               float* lse, int B, int H, int N, int d, float scale,
               int causal, hipStream_t stream);

/*
 * Key-split attention forward (bf16), for grids too small to fill the GPU
 * and for decode-shaped calls.  The keys of every query tile are cut into
 * `num_splits` chunks handled by separate workgroups; each writes its own
 * normalised O and LSE to `workspace`, and a merge kernel combines them with
 * LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s -- the
 * online-softmax merge applied to whole chunks, as FlashDecoding does for
 * decoding (zzszmyf.github.io notes "FlashAttention 原理是什么", sections 5
 * and 12.1).  Results equal fa_fwd's up to rounding order.
 *   q, o      : [B,H,Nq,d] bf16;  k, v : [B,H,Nk,d] bf16;  lse : [B,H,Nq] fp32.
 *   Nq, Nk    : query rows and keys, >= 1.  Causal aligns the last query with
 *               the last key: query i attends keys j <= i + Nk - Nq, so causal
 *               calls need Nq <= Nk (Nq == Nk is the square problem).
 *   num_splits: 1..256 chunks (fa_fwd_splitkv_num_splits suggests one).
 *   workspace : device buffer of at least fa_fwd_splitkv_workspace_size(...)
 *               bytes, 16-byte aligned, owned by the caller, overlapping no
 *               other argument; its contents are scratch (nothing is kept
 *               between calls, and calls sharing one workspace must not run
 *               concurrently).
 * Errors as for fa_fwd, plus FA_ERR_SHAPE for causal with Nq > Nk or when
 * num_splits * B * H * ceil(Nq/128) reaches 2^24 (the key-split launch runs
 * that many 256-thread workgroups), FA_ERR_SPLITS and FA_ERR_WORKSPACE.  With num_splits > 1 two kernels are
 * queued on `stream`; with num_splits == 1 the single-pass kernel writes O
 * and LSE directly (the workspace is still required and left untouched).
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal,
                   int num_splits, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/* Bytes of workspace fa_fwd_splitkv needs for these sizes; 0 if an
 * argument is out of range.  Host only, no HIP call. */
size_t fa_fwd_splitkv_workspace_size(int B, int H, int Nq, int d, int num_splits);

/* A chunk count for a GPU with num_cus compute units (<= 0 means 256): two
 * workgroups per CU when chunks keep at least sixteen 64-key tiles (up to
 * four per CU while they still do); else, if that takes at most 128 chunks,
 * two per CU with chunks of at least 4 tiles; else one per CU with chunks of
 * 8 tiles, or of 4 when the keys are fewer.  Host only, no HIP call. */
int fa_fwd_splitkv_num_splits(int B, int H, int Nq, int Nk, int num_cus);

/*
 * fa_fwd_splitkv without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The call allocates nothing: the
 * fp32 key-split partials go to a static device array owned by the library,
 * fa_fwd_splitkv_noalloc_max_bytes() bytes (32 MiB) on each GPU the library
 * has been loaded on, held until the process ends.  Its device address is
 * looked up once per GPU (on the first call for that GPU, with the stream's
 * GPU made current for the lookup) and cached.
 *   Arguments, layout and results as for fa_fwd_splitkv with the same
 *   num_splits (the same kernels run, so the outputs are bit-identical).
 *   Errors as for fa_fwd_splitkv, except that FA_ERR_WORKSPACE cannot occur;
 *   FA_ERR_SCRATCH when fa_fwd_splitkv_workspace_size(B, H, Nq, d,
 *   num_splits) exceeds fa_fwd_splitkv_noalloc_max_bytes() (checked on the
 *   host before any HIP call); FA_ERR_HIP if the scratch lookup or a launch
 *   fails.
 * Every call on one GPU shares that GPU's scratch and nothing in it is kept
 * from one call to the next (every partial is written before it is read):
 * calls that overlap in time on one GPU (two streams, or two host threads)
 * race on it and must be serialised by the caller.
 */
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Nq, int Nk, int d, float scale, int causal,
                           int num_splits, hipStream_t stream);

/* Size in bytes of the static scratch of fa_fwd_splitkv_noalloc.  Host only. */
size_t fa_fwd_splitkv_noalloc_max_bytes(void);

/*
 * Attention forward with grouped K/V heads (bf16): multi-query and
 * grouped-query attention, the variants that cut K/V reads (aiqz.cc Flash
 * Attention IO article, section 性能调优经验).  Query head h of batch b reads
 * K/V head h / (H / Hkv) of batch b; Hkv == H is ordinary multi-head
 * attention, Hkv == 1 multi-query attention.
 *   q, o      : [B,H,Nq,d] bf16;  k, v : [B,Hkv,Nk,d] bf16;  lse : [B,H,Nq] fp32.
 *   H, Hkv    : query heads and K/V heads, Hkv >= 1 dividing H.
 *   Nq, Nk    : query rows and keys per head, >= 1; causal aligns the last
 *               query with the last key (query i sees keys j <= i + Nk - Nq)
 *               and needs Nq <= Nk.  The H/Hkv query heads of a K/V head
 *               must hold fewer than 2^31 rows together.
 *   num_splits: 1 -> one pass, O and LSE written directly, workspace ignored
 *               (may be NULL); 2..256 -> the keys are cut into chunks merged
 *               as in fa_fwd_splitkv, with a workspace of at least
 *               fa_fwd_splitkv_workspace_size(B, H, Nq, d, num_splits) bytes
 *               (the partials are per query row).
 * The query heads sharing a K/V head are processed together: short query
 * blocks (decoding) are packed into one tile, so K/V is read once per K/V
 * head rather than once per query head.  Results equal those of fa_fwd_splitkv
 * on K/V with every head repeated H/Hkv times, up to rounding order.
 * Errors as for fa_fwd_splitkv (its workgroup bound counts the 128-row
 * query tiles of each K/V head's packed rows), plus FA_ERR_HEADS.
 */
int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
               int num_splits, void* workspace, size_t workspace_bytes,
               hipStream_t stream);

/* A chunk count for fa_fwd_gqa, chosen as fa_fwd_splitkv_num_splits does
 * (1 if an argument is out of range).  Host only, no HIP call. */
int fa_fwd_gqa_num_splits(int B, int H, int Hkv, int Nq, int Nk, int causal, int num_cus);

/*
 * Attention backward (bf16), by recomputation: the gradients of
 * O = softmax(scale * Q K^T) V for an upstream gradient dO, rebuilt from Q,
 * K, V and the forward pass's O and LSE without any N x N buffer
 * (zzszmyf.github.io notes "FlashAttention 原理是什么", section 6; aiqz.cc
 * Flash Attention IO article, section 工程实现细节).  With P_ij =
 * exp(scale <q_i, k_j> - LSE_i) over the visible pairs,
 *     dV = P^T dO,  dS = P * (dO V^T - D),  D_i = <dO_i, O_i>,
 *     dQ = scale dS K,  dK = scale dS^T Q.
 *   q, k, v, o, dout : device pointers, [B,H,N,d] bf16 (o and lse as written
 *                      by fa_fwd for the same q, k, v, scale and causal).
 *   lse              : [B,H,N] fp32.
 *   dq, dk, dv       : [B,H,N,d] bf16, written (round to nearest even).
 *   workspace        : device buffer of at least fa_bwd_workspace_size(...)
 *                      bytes, 16-byte aligned; scratch for the per-row D.
 *   B, H, N, d, scale, causal : as for fa_fwd.
 * dq, dk, dv and the workspace must not overlap each other or any input.
 * Two kernels are queued on `stream` (dQ with D, then dK and dV); neither
 * uses atomics, so results are reproducible bit for bit.  Errors as for
 * fa_fwd, plus FA_ERR_WORKSPACE.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
           float scale, int causal, void* workspace, size_t workspace_bytes,
           hipStream_t stream);

/* Bytes of workspace fa_bwd needs (0 if an argument is out of range).
 * Host only, no HIP call. */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/*
 * Backward pass with grouped K/V heads (MQA/GQA, as fa_fwd_gqa with
 * Nq = Nk = N): q, o, dout, dq are [B,H,N,d] bf16, lse [B,H,N] fp32, and
 * k, v, dk, dv are [B,Hkv,N,d] bf16, query head h of batch b reading K/V head
 * h / (H / Hkv) of batch b.  Since a shared K/V head enters the forward once
 * per query head of its group, its gradient is the sum of the per-head
 * gradients (the chain rule through the copies): each query head's fp32
 * dK and dV go to the workspace and a third kernel sums every group in head
 * order and rounds to bf16, so results stay reproducible bit for bit.
 *   workspace : at least fa_bwd_gqa_workspace_size(B, H, Hkv, N, d) bytes,
 *               16-byte aligned; Hkv == H needs only fa_bwd's workspace and
 *               gives exactly fa_bwd's results.
 * Other arguments and errors as for fa_bwd, plus FA_ERR_HEADS when Hkv does
 * not divide H.
 */
int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
               float scale, int causal, void* workspace, size_t workspace_bytes,
               hipStream_t stream);

/* Bytes of workspace fa_bwd_gqa needs (0 if an argument is out of range).
 * Host only, no HIP call. */
size_t fa_bwd_gqa_workspace_size(int B, int H, int Hkv, int N, int d);

/*
 * fp8 forward with per-block scales: the low-precision variant of the method
 * (zzszmyf.github.io notes "FlashAttention 原理是什么", section 10 item ③ and
 * section 12.2: block-wise quantization with one scale per block).  Inputs
 * are quantized to OCP E4M3 codes in the MX block layout that gfx950's
 * matrix cores consume: every 32 consecutive elements along a contracted
 * dimension share one E8M0 scale byte E (value 2^(E-127)).  For a block with
 * largest magnitude amax = m * 2^f (1 <= m < 2) the scale exponent is
 * X = f - 8 if m <= 1.75 else f - 7 (the smallest X with amax <= 448 * 2^X),
 * E = clamp(X + 127, 0, 254) (E = 0 for a zero or subnormal amax), and each
 * code is the round-to-nearest-even E4M3 value of x * 2^(127 - E); nothing
 * is clipped.  The dequantized input is decode(code) * 2^(E - 127).
 *
 * fa_quantize_qk_fp8: Q or K rows.  x bf16 [rows, d] (device) -> x8 codes
 *   [rows, d] (one byte each) and xs scales [rows, d/32] (block c covers
 *   dims 32c .. 32c+31).  rows >= 1, d in {64, 128}, rows * d/32 below
 *   2^32 (one thread per block).
 * fa_quantize_v_fp8: V of BH = B*H heads.  v bf16 [BH, N, d] -> v8t codes in
 *   fa_fp8_v_bytes(BH, N, d) bytes and vs scales in
 *   fa_fp8_v_scale_bytes(BH, N, d) bytes.  Blocks are 32 consecutive keys of
 *   one head dim.  Layout: T = ceil(N/64) tiles of 64 keys per head; v8t is
 *   [BH, T, d, 64] (each tile transposed, keys past N zero) with position
 *   32h + j (h in {0,1}, j in 0..31) of a tile row holding key
 *   32*(j/16) + (j%4) + 8*((j%16)/4) + 4h of the tile; vs is [BH, T, 2, 32,
 *   d/32], element (t, b, i, c) the scale of keys 64t + 32b .. +31 of head
 *   dim 32c + i.  BH * T * 2d must stay below 2^32 (threads of the launch).
 * fa_fwd_fp8: attention of the dequantized inputs.  q8, qs, k8, ks as
 *   written by fa_quantize_qk_fp8 for the [B*H*N, d] rows of Q and K; v8t,
 *   vs by fa_quantize_v_fp8 for V; o bf16 [B,H,N,d] and lse fp32 [B,H,N]
 *   written as by fa_fwd (same scale and causal arguments).  Scores and the
 *   products with V run on fp8 matrix cores with fp32 accumulation; the
 *   softmax is fp32 and the probabilities are rounded to E4M3 (values at
 *   most 2^8) for the product with V, the row sums taken over the same
 *   rounded values.
 * All pointers are device pointers, 16-byte aligned; outputs must not overlap
 * inputs.  Errors as for fa_fwd.  Each call queues one kernel on `stream`.
 */
int fa_quantize_qk_fp8(const void* x, int64_t rows, int d, void* x8, void* xs, hipStream_t stream);
int fa_quantize_v_fp8(const void* v, int BH, int N, int d, void* v8t, void* vs, hipStream_t stream);
size_t fa_fp8_v_bytes(int BH, int N, int d);        /* 0 if out of range; host only */
size_t fa_fp8_v_scale_bytes(int BH, int N, int d);  /* 0 if out of range; host only */
int fa_fwd_fp8(const void* q8, const void* qs, const void* k8, const void* ks, const void* v8t,
               const void* vs, void* o, float* lse, int B, int H, int N, int d, float scale,
               int causal, hipStream_t stream);

/*
 * Rotated quantization of Q or K rows (incoherent processing: the notes page
 * "FlashAttention 原理是什么", sections 10 item ③ and 12.2, pairs block
 * quantization with an orthogonal transform that spreads outlier channels
 * over all head dims before rounding, since Q R (K R)^T = Q K^T for
 * orthogonal R).  Each row x is replaced by x diag(s) H_d, with H_d the
 * Sylvester-Hadamard matrix of order d (H_1 = [1], H_2n = [[H_n, H_n],
 * [H_n, -H_n]]; entries +-1, H H^T = d I) and s a sign per head dim, then
 * quantized exactly as fa_quantize_qk_fp8 does.  The transform is computed
 * exactly in double precision (exact while the magnitudes of a row span less
 * than 2^38) and rounded once to float before the block scales are chosen;
 * an exact zero is +0 (code 0x00).
 *   signs : device pointer to d bytes, entry c < 0 flips head dim c; NULL
 *           for no flips.  Q and K must be rotated with the same signs.
 * Since (Q R)(K R)^T = d Q K^T, attention over rotated Q and K is
 * fa_fwd_fp8 (or fa_fwd_fp8_gqa) with scale / d (d a power of two, so the
 * division is exact); V is not rotated.  Other arguments, layout and errors
 * as for fa_quantize_qk_fp8 (the signs must not overlap x8 or xs).
 */
int fa_quantize_qk_fp8_rotated(const void* x, int64_t rows, int d, const signed char* signs,
                               void* x8, void* xs, hipStream_t stream);

/*
 * fp8 forward with grouped K/V heads (MQA/GQA, as fa_fwd_gqa with
 * Nq = Nk = N): q8, qs for the [B*H*N, d] rows of Q; k8, ks for the
 * [B*Hkv*N, d] rows of K and v8t, vs for the B*Hkv heads of V, as the
 * quantizers write them; query head h of batch b reads K/V head
 * h / (H / Hkv) of batch b.  Hkv == H is fa_fwd_fp8.  Errors as for
 * fa_fwd_fp8, plus FA_ERR_HEADS when Hkv does not divide H.
 */
int fa_fwd_fp8_gqa(const void* q8, const void* qs, const void* k8, const void* ks, const void* v8t,
                   const void* vs, void* o, float* lse, int B, int H, int Hkv, int N, int d,
                   float scale, int causal, hipStream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
