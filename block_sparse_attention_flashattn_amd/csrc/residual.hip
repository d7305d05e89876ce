// Dense-sparse residual compensation: the two elementwise passes.
//
// Page "Can sparse attention close the quality gap in diffusion transformers"
// (MC-Sparse summary), section on residual compensation: at an anchor step the
// residual between the dense and the sparse attention outputs is recorded; at a
// reuse step the cached residual is added to the sparse output (the anchor's
// selection is reused too, per the section on reusing exact selection).
//   residual:   R = O_dense - O_sparse
//   compensate: O = O_sparse + R
// bf16 in and out, the difference or sum formed in fp32 and rounded once (RNE).
// Memory-bound: 16-byte accesses, grid-stride over 8-element groups.
#include "common.h"

namespace bsa {
namespace {

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf2f(unsigned short h) { return __uint_as_float(uint32_t(h) << 16); }
__device__ __forceinline__ unsigned short f2bf(float f) {
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(f));
}

template <bool SUB>
__global__ __launch_bounds__(256) void elementwise_kernel(const uint16_t* __restrict__ a,
                                                          const uint16_t* __restrict__ b,
                                                          uint16_t* __restrict__ out, int64_t n) {
  const int64_t n8 = n / 8;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t g = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; g < n8; g += stride) {
    const u16x8 x = reinterpret_cast<const u16x8*>(a)[g];
    const u16x8 y = reinterpret_cast<const u16x8*>(b)[g];
    u16x8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = f2bf(SUB ? bf2f(x[e]) - bf2f(y[e]) : bf2f(x[e]) + bf2f(y[e]));
    reinterpret_cast<u16x8*>(out)[g] = z;
  }
  // The last n % 8 elements.
  if (blockIdx.x == 0 && int64_t(threadIdx.x) < n - 8 * n8) {
    const int64_t t = 8 * n8 + threadIdx.x;
    out[t] = f2bf(SUB ? bf2f(a[t]) - bf2f(b[t]) : bf2f(a[t]) + bf2f(b[t]));
  }
}

template <bool SUB>
bsa_status launch(const void* a, const void* b, void* out, int64_t n, void* stream) {
  if (!a || !b || !out || n < 0) return BSA_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(b) || !aligned16(out)) return BSA_ERR_INVALID_ARG;
  if (n == 0) return BSA_OK;
  const int64_t groups = (n + 7) / 8;
  const int64_t blocks = (groups + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 8192 ? blocks : 8192);
  hipLaunchKernelGGL(elementwise_kernel<SUB>, dim3(grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(a),
                     static_cast<const uint16_t*>(b), static_cast<uint16_t*>(out), n);
  BSA_HIP_CHECK_LAUNCH();
  return BSA_OK;
}

}  // namespace
}  // namespace bsa

extern "C" BSA_API bsa_status bsa_residual(const void* o_dense, const void* o_sparse, void* r_out,
                                           int64_t n, void* stream) {
  return bsa::launch<true>(o_dense, o_sparse, r_out, n, stream);
}

extern "C" BSA_API bsa_status bsa_compensate(const void* o_sparse, const void* r, void* o_out,
                                             int64_t n, void* stream) {
  return bsa::launch<false>(o_sparse, r, o_out, n, stream);
}
