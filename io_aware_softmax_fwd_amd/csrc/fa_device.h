// Device-side helpers shared by the bf16 attention kernels (forward and
// backward): vector types of the gfx950 MFMA operands, bf16 packing, the
// cross-half reductions of a 64-lane wave and the LDS-DMA addressing of a
// padded K/V-style tile.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;

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

// Block b -> (head, rank of the block among its head's per blocks).  hg > 0
// needs BH a multiple of 8: blocks are dealt to the eight XCDs in turn (block
// b to XCD b % 8), each with its own L2, so head h is placed on XCD h % 8 and
// an XCD takes its heads hg at a time, rank 0 of every head of the group
// first, then rank 1, ...  The blocks of a group then read the same K/V at
// about the same time and share it in L2.  hg = 0: heads vary fastest.
__device__ __forceinline__ void xcd_order(int b, int BH, int per, int hg, int& head, int& rank) {
  if (hg > 0) {
    const int xcd = b & 7, s = b >> 3;
    const int grp = s / (hg * per), r = s % (hg * per);
    head = xcd + 8 * (grp * hg + r % hg);
    rank = r / hg;
  } else {
    head = b % BH;
    rank = b / BH;
  }
}

}  // namespace
}  // namespace fa
