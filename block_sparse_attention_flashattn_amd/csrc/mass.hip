// Exact attention mass per block pair, and the mass a CSR keeps.
//
// Page "Can sparse attention close the quality gap in diffusion transformers"
// (MC-Sparse summary): its oracle sections compare sparse attention, at equal
// density, with oracles that keep the most mass of the exact dense attention
// probabilities (the block oracle picks KV blocks per query block); its section
// on token-level selection notes that exact selection needs the scores, which a
// FlashAttention pass does not expose, so it takes two passes.  The first pass
// is the dense forward (its LSE); this file is the second:
//
//   mass[r, j] = sum over queries t of block i and keys c of block j (t, c < N)
//                of exp(scale q_t.k_c - lse_t),
//
// r = (bi*H + h)*nb + i, i.e. the block sums of the dense probabilities.  The
// oracle selection itself reuses the mask builder's row selection (mask.hip).
#include "common.h"

namespace bsa {
namespace {

constexpr int kMassBlocksPerWg = 8;  // KV blocks per workgroup

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           0x00020000);
}

__device__ __forceinline__ bf16x8 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// One workgroup (four wavefronts) per (query block, group of KV blocks).  A block
// pair is cut into (BLK/32)^2 tiles of 32 keys x 32 queries, S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16: lane (ql, hh) holds, for query ql of its tile, the
// keys 8(e/4) + 4hh + (e%4), e = 0..15.  A wavefront owns BLK*BLK/4096 tiles that
// share one key group (BLK 64: one query group; BLK 128: all four), keeps their
// query fragments in registers and reads its key fragments straight from memory
// (16-byte buffer loads; rows past N read as zeros and are masked out).
template <int BLK, int HD>
__global__ __launch_bounds__(256) void mass_kernel(const uint16_t* __restrict__ Q,
                                                   const uint16_t* __restrict__ K,
                                                   const float* __restrict__ lse, int32_t N,
                                                   int32_t nb, float sl2,
                                                   float* __restrict__ mass) {
  constexpr int QG = BLK / 32;
  constexpr int PW = QG * QG / 4;  // tiles per wavefront
  constexpr int NC = HD / 16;      // 16-deep MFMA steps
  __shared__ float red[4][kMassBlocksPerWg];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ql = lane & 31, hh = lane >> 5;
  const int r = blockIdx.x;
  const int bh = r / nb, i = r - bh * nb;
  const int j0 = blockIdx.y * kMassBlocksPerWg;
  const int jn = min(kMassBlocksPerWg, nb - j0);
  const size_t head = size_t(bh) * size_t(N) * HD;
  const uint32_t hbytes = static_cast<uint32_t>(N) * HD * 2u;
  const __amdgpu_buffer_rsrc_t qr = rsrc(Q + head, hbytes);
  const __amdgpu_buffer_rsrc_t kr = rsrc(K + head, hbytes);
  const int kg = (wave * PW) / QG;  // the key group of all this wavefront's tiles

  bf16x8 qf[PW][NC];
  float lq[PW];   // lse of the lane's query in log2 units
  bool qv[PW];    // the query exists and has a finite normaliser
#pragma unroll
  for (int t = 0; t < PW; ++t) {
    const int qg = (wave * PW + t) % QG;
    const int qrow = i * BLK + 32 * qg + ql;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[t][c] = load16(qr, static_cast<uint32_t>(qrow * HD + 16 * c + 8 * hh) * 2u);
    const float l = qrow < N ? lse[size_t(bh) * N + qrow] : -INFINITY;
    qv[t] = l > -INFINITY && l < INFINITY;
    lq[t] = qv[t] ? l * 1.4426950408889634f : 0.f;
  }

  for (int jj = 0; jj < jn; ++jj) {
    const int j = j0 + jj;
    const int krow = j * BLK + 32 * kg + ql;
    bf16x8 kf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
      kf[c] = load16(kr, static_cast<uint32_t>(krow * HD + 16 * c + 8 * hh) * 2u);
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < PW; ++t) {
      f32x16 s = {};
#pragma unroll
      for (int c = 0; c < NC; ++c) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c], qf[t][c], s, 0, 0, 0);
      if (qv[t]) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = j * BLK + 32 * kg + 8 * (e >> 2) + 4 * hh + (e & 3);
          if (key < N) sum += __builtin_amdgcn_exp2f(s[e] * sl2 - lq[t]);
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane == 0) red[wave][jj] = sum;
  }
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < jn) {
    const int t = threadIdx.x;
    mass[size_t(r) * nb + j0 + t] = (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
  }
}

// One thread per CSR row: the mass of its listed blocks, in list order.
__global__ __launch_bounds__(256) void csr_mass_kernel(const float* __restrict__ mass,
                                                       int32_t n_rows, int32_t nb,
                                                       const int32_t* __restrict__ row_ptr,
                                                       const int32_t* __restrict__ col_idx,
                                                       float* __restrict__ out) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= n_rows) return;
  const int nnz = row_ptr[n_rows];
  const int b = min(max(row_ptr[r], 0), nnz);
  const int e = min(max(row_ptr[r + 1], b), nnz);
  float s = 0.f;
  for (int c = b; c < e; ++c) {
    const int j = col_idx[c];
    if (j >= 0 && j < nb) s += mass[size_t(r) * nb + j];
  }
  out[r] = s;
}

template <int BLK, int HD>
bsa_status launch_mass(const void* q, const void* k, const float* lse, int32_t n_rows, int32_t N,
                       int32_t nb, float sl2, float* mass, hipStream_t s) {
  const dim3 grid(n_rows, (nb + kMassBlocksPerWg - 1) / kMassBlocksPerWg);
  hipLaunchKernelGGL((mass_kernel<BLK, HD>), grid, dim3(256), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), lse, N, nb,
                     sl2, mass);
  BSA_HIP_CHECK_LAUNCH();
  return BSA_OK;
}

}  // namespace
}  // namespace bsa

extern "C" BSA_API bsa_status bsa_block_mass(const void* q, const void* k, const float* lse,
                                             int32_t B, int32_t H, int32_t N, int32_t D,
                                             int32_t block, float scale, float* mass_out,
                                             void* stream) {
  using namespace bsa;
  if (!q || !k || !lse || !mass_out) return BSA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || !(scale == scale)) return BSA_ERR_INVALID_ARG;
  if (!supported_shape(D, block)) return BSA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k)) return BSA_ERR_INVALID_ARG;
  // Buffer offsets inside one head are 32-bit.
  if (int64_t(N) * D * 2 >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  const int32_t nb = n_blocks(N, block);
  const int64_t rows = int64_t(B) * H * nb;
  if (rows > INT32_MAX - 1 || rows * nb > (int64_t(1) << 40)) return BSA_ERR_UNSUPPORTED;
  const float sc = scale > 0.f ? scale : 1.f / sqrtf(static_cast<float>(D));
  const float sl2 = sc * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t n = static_cast<int32_t>(rows);
  if (block == 64 && D == 64) return launch_mass<64, 64>(q, k, lse, n, N, nb, sl2, mass_out, s);
  if (block == 64 && D == 128) return launch_mass<64, 128>(q, k, lse, n, N, nb, sl2, mass_out, s);
  if (block == 128 && D == 64) return launch_mass<128, 64>(q, k, lse, n, N, nb, sl2, mass_out, s);
  return launch_mass<128, 128>(q, k, lse, n, N, nb, sl2, mass_out, s);
}

extern "C" BSA_API bsa_status bsa_csr_mass(const float* mass, int32_t n_rows, int32_t nb,
                                           const int32_t* row_ptr, const int32_t* col_idx,
                                           float* out, void* stream) {
  if (!mass || !row_ptr || !col_idx || !out || n_rows < 1 || nb < 1) return BSA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(bsa::csr_mass_kernel, dim3((n_rows + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), mass, n_rows, nb, row_ptr, col_idx, out);
  BSA_HIP_CHECK_LAUNCH();
  return BSA_OK;
}
