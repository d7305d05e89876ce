// Internal helpers shared by the libbsa translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa.h"

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxBlocks = 1024;  // nb limit of the mask builder (16 columns per lane)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool supported_shape(int32_t D, int32_t block) {
  return (D == 64 || D == 128) && (block == 64 || block == 128);
}

inline int32_t n_blocks(int32_t N, int32_t block) { return (N + block - 1) / block; }

}  // namespace bsa

#define BSA_HIP_CHECK_LAUNCH()                              \
  do {                                                      \
    if (hipGetLastError() != hipSuccess) return BSA_ERR_HIP; \
  } while (0)
