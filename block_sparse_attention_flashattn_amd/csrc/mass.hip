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

// One workgroup (four wavefronts) per (four 32-query groups of one head: two query
// blocks at BLK 64, one at BLK 128; a group of KV blocks).  A block pair is cut
// into tiles of 32 keys x 32 queries, S^T = K Q^T with v_mfma_f32_32x32x16_bf16:
// lane (ql, hh) holds, for query ql of the tile, the keys 8(e/4) + 4hh + (e%4),
// e = 0..15.  Each wavefront takes one 32-key group of a KV block against all four
// query groups (whose fragments stay in registers), so every key fragment is read
// once per workgroup and serves 128 queries, straight from memory (16-byte buffer
// loads; rows past N read as zeros and are masked out); the four wavefronts cover
// 128 keys per step (two KV blocks at BLK 64, one at BLK 128).  Per-lane partial
// sums are kept per (query block, KV block) and reduced across the wavefront once
// at the end.
template <int BLK, int HD>
__global__ __launch_bounds__(256) void mass_kernel(const uint16_t* __restrict__ Q,
                                                   const uint16_t* __restrict__ K,
                                                   const float* __restrict__ lse, int32_t N,
                                                   int32_t nb, float sl2,
                                                   float* __restrict__ mass) {
  constexpr int QG = BLK / 32;                // 32-row groups per block
  constexpr int QB = 4 / QG;                  // query blocks per workgroup
  constexpr int NC = HD / 16;                 // 16-deep MFMA steps
  constexpr int JPS = 4 / QG;                 // KV blocks per step
  constexpr int NS = kMassBlocksPerWg / JPS;  // steps
  __shared__ float red[QB][4][kMassBlocksPerWg];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ql = lane & 31, hh = lane >> 5;
  const int npair = (nb + QB - 1) / QB;       // query-block tuples per head
  const int bh = blockIdx.x / npair;
  const int i0 = (blockIdx.x - bh * npair) * QB;
  const int j0 = blockIdx.y * kMassBlocksPerWg;
  const int jn = min(kMassBlocksPerWg, nb - j0);
  const size_t head = size_t(bh) * size_t(N) * HD;
  const uint32_t hbytes = static_cast<uint32_t>(N) * HD * 2u;
  const __amdgpu_buffer_rsrc_t qr = rsrc(Q + head, hbytes);
  const __amdgpu_buffer_rsrc_t kr = rsrc(K + head, hbytes);
  const int kg = wave % QG;    // key group of this wavefront
  const int jsub = wave / QG;  // which KV block of a step

  // Query group g = 0..3: block i0 + g / QG, rows 32 (g % QG) .. +31.
  bf16x8 qf[4][NC];
  float lq[4];  // lse of the lane's query in log2 units; +inf drops the query
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int qb = i0 + g / QG;
    const int qrow = qb * BLK + 32 * (g % QG) + ql;
    const bool ok = qb < nb && qrow < N;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[g][c] = load16(qr, ok ? static_cast<uint32_t>(qrow * HD + 16 * c + 8 * hh) * 2u : hbytes);
    const float l = ok ? lse[size_t(bh) * N + qrow] : -INFINITY;
    lq[g] = (l > -INFINITY && l < INFINITY) ? l * 1.4426950408889634f : INFINITY;
  }

  // The next step's K rows are requested before this step computes; steps past
  // the workgroup's blocks read zeros (out-of-range offsets), so no load sits
  // behind a branch and its own wait.
  auto fetch = [&](int t, bf16x8* dst) {
    const int jj = t * JPS + jsub;
    const int kbase = (j0 + jj) * BLK + 32 * kg;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      dst[c] = load16(kr, t < NS && jj < jn
                              ? static_cast<uint32_t>((kbase + ql) * HD + 16 * c + 8 * hh) * 2u
                              : hbytes);
  };
  bf16x8 kbuf[2][NC];
  fetch(0, kbuf[0]);
  float part[QB][NS];
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    fetch(t + 1, kbuf[(t + 1) & 1]);
#pragma unroll
    for (int b = 0; b < QB; ++b) part[b][t] = 0.f;
    const int jj = t * JPS + jsub;
    if (jj < jn) {
      const int j = j0 + jj;
      const int kbase = j * BLK + 32 * kg;
      const bf16x8* kf = kbuf[t & 1];
      const bool full = kbase + 32 <= N;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x16 sv = {};
#pragma unroll
        for (int c = 0; c < NC; ++c)
          sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c], qf[g][c], sv, 0, 0, 0);
        float a0 = 0.f, a1 = 0.f;
        if (full) {
#pragma unroll
          for (int e = 0; e < 16; e += 2) {
            a0 += __builtin_amdgcn_exp2f(fmaf(sv[e], sl2, -lq[g]));
            a1 += __builtin_amdgcn_exp2f(fmaf(sv[e + 1], sl2, -lq[g]));
          }
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kbase + 8 * (e >> 2) + 4 * hh + (e & 3);
            if (key < N) a0 += __builtin_amdgcn_exp2f(fmaf(sv[e], sl2, -lq[g]));
          }
        }
        part[g / QG][t] += a0 + a1;
      }
    }
  }
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      float v = part[b][t];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      const int jj = t * JPS + jsub;
      if (lane == 0 && jj < jn) red[b][kg][jj] = v;
    }
  __syncthreads();
  const int t = threadIdx.x % kMassBlocksPerWg;
  const int b = threadIdx.x / kMassBlocksPerWg;
  if (b < QB && t < jn && i0 + b < nb) {
    float m = red[b][0][t];
#pragma unroll
    for (int g = 1; g < QG; ++g) m += red[b][g][t];
    mass[(size_t(bh) * nb + i0 + b) * nb + j0 + t] = m;
  }
}

// One wavefront per CSR row: the mass of its listed blocks (each lane sums every
// 64th entry of the row, then the lanes' sums are added by shuffles), so a row's
// column and mass loads are all in flight at once.
__global__ __launch_bounds__(256) void csr_mass_kernel(const float* __restrict__ mass,
                                                       int32_t n_rows, int32_t nb,
                                                       const int32_t* __restrict__ row_ptr,
                                                       const int32_t* __restrict__ col_idx,
                                                       float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  const int nnz = row_ptr[n_rows];
  const int b = min(max(row_ptr[r], 0), nnz);
  const int e = min(max(row_ptr[r + 1], b), nnz);
  float s = 0.f;
  for (int c = b + lane; c < e; c += 64) {
    const int j = col_idx[c];
    if (j >= 0 && j < nb) s += mass[size_t(r) * nb + j];
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) s += __shfl_xor(s, d);
  if (lane == 0) out[r] = s;
}

template <int BLK, int HD>
bsa_status launch_mass(const void* q, const void* k, const float* lse, int32_t n_rows, int32_t N,
                       int32_t nb, float sl2, float* mass, hipStream_t s) {
  constexpr int QB = 128 / BLK;  // query blocks per workgroup
  const int64_t heads = n_rows / nb;
  const dim3 grid(static_cast<uint32_t>(heads * ((nb + QB - 1) / QB)),
                  (nb + kMassBlocksPerWg - 1) / kMassBlocksPerWg);
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
  hipLaunchKernelGGL(bsa::csr_mass_kernel, dim3((n_rows + 3) / 4), dim3(256), 0,
                     static_cast<hipStream_t>(stream), mass, n_rows, nb, row_ptr, col_idx, out);
  BSA_HIP_CHECK_LAUNCH();
  return BSA_OK;
}
