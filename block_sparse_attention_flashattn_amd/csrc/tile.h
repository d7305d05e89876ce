// Device helpers shared by the attention kernels (forward, gathered forward,
// backward): tile swizzle, bf16 packing, buffer descriptors, LDS reads, and the
// running-max conventions.
#pragma once
#include "common.h"

namespace bsa {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
#define BSA_LDS __attribute__((address_space(3)))

// Swizzle of the 16-byte chunks of tile row r (64 banks of 4 bytes; a
// 16-byte read serves 16 lanes per cycle, an 8-byte read 32 lanes).
//  * 128-byte rows (D = 64): a bank group is 8 (r & 1) + chunk.  Reversing the
//    bits of (r >> 1) & 7 gives the 8 same-parity rows of any aligned 16-row
//    group distinct chunks (16 lanes reading one logical chunk of 16 rows), and
//    rows r, r + 2 of an aligned 4-row group different aligned 4-chunk blocks
//    (the transposing V read: 4 rows x 4 chunks per half-wave).
//  * 256-byte rows (D = 128): a bank group is the chunk.  Swapping the two
//    2-bit fields of r & 15 is a bijection on 16 rows and sends the 4 rows of an
//    aligned 4-row group to 4 different aligned 4-chunk blocks.
template <int ROWB>
__device__ __forceinline__ int chunk_swizzle(int r) {
  if constexpr (ROWB == 128) {
    const int m = (r >> 1) & 7;
    return ((m & 1) << 2) | (m & 2) | ((m >> 2) & 1);
  } else {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  }
}

// Byte offset of the 16-byte chunk c of row r inside a swizzled tile.
template <int ROWB>
__device__ __forceinline__ uint32_t swz(int r, int c) {
  return uint32_t(r) * ROWB + uint32_t((c ^ chunk_swizzle<ROWB>(r)) << 4);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const uint16_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
  const uint16_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(b));
  return uint32_t(lo) | (uint32_t(hi) << 16);
}

// The two bf16 values packed in a 32-bit word, widened to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           0x00020000);
}

// Value of lane l ^ 32 (the other half of the wavefront), without LDS.
__device__ __forceinline__ float other_half(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  // Lanes < 32 receive the upper half in the second result, lanes >= 32 the
  // lower half in the first.
  return __uint_as_float((threadIdx.x & 32) ? sw[0] : sw[1]);
}

__device__ __forceinline__ v4s lds_read_tr(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((BSA_LDS v4s*)(static_cast<uintptr_t>(addr)));
}

__device__ __forceinline__ bf16x8 lds_read16(uint32_t addr) {
  return *((const BSA_LDS bf16x8*)(static_cast<uintptr_t>(addr)));
}

// Running-max start value of the wide kernel: finite, so that it can enter the
// exponent argument directly (scores of -inf still give exp2 = 0), and far
// below any score.
constexpr float kNoMax = -1.0e30f;

// IEEE maximum (NaN-propagating): lowers to v_maximum3_f32 chains with no
// NaN-quieting copies in front, unlike fmaxf.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

}  // namespace bsa
