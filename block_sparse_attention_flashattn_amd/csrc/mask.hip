// Mean-pool top-k block-mask builder for gfx950.
//
// MC-Sparse summary, section on mean-pooled block scoring: the naive selector
// represents each query block and each KV block by the mean of its tokens,
// scores every pair by the dot product of the two means and keeps the best
// KV blocks per query block at the target density.  BSA-DiT §2.3 unions that
// with a static prior; BSA-DiT §5.3 lets each query block have its own count;
// BSA-DiT §5.3 (last paragraph) asks that the dynamic part run on the GPU so
// no index crosses PCIe per step.
//
// Three launches on one stream:
//   pool    one workgroup per (head, block, Q|K): 16-byte coalesced loads,
//           fp32 sums over the valid tokens, LDS reduction, divide by count.
//   score   32x32 output tiles of Pq Pk^T per head from LDS, fp32 FMA.
//   select  one wavefront per CSR row: prior/diagonal flags, then `fill`
//           rounds of a wavefront-wide 64-bit argmax over (score, -column)
//           keys, then a ballot/mbcnt compaction that writes the row's
//           columns in ascending order at row_ptr[r].
#include <math.h>

#include "common.h"

namespace bsa {
namespace {

constexpr int kStatusBytes = 256;

__global__ void zero_status_kernel(int32_t* status) { *status = 0; }

template <int HD>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ Q,
                                                   const uint16_t* __restrict__ K, int32_t N,
                                                   int32_t nb, int32_t block,
                                                   float* __restrict__ Pq,
                                                   float* __restrict__ Pk,
                                                   int32_t* __restrict__ status) {
  // The builder's status word (counted up by select_kernel, which runs after
  // this launch) starts at zero.
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *status = 0;
  constexpr int CPR = HD / 8;     // 16-byte chunks per token row
  constexpr int RPP = 256 / CPR;  // token rows per pass
  __shared__ float red[RPP][HD + 1];
  const int tid = threadIdx.x;
  const int blk = blockIdx.x;  // (bh, i) flattened
  const int bh = blk / nb;
  const int i = blk - bh * nb;
  const int valid = min(block, N - i * block);
  const uint16_t* X = blockIdx.y == 0 ? Q : K;
  float* P = blockIdx.y == 0 ? Pq : Pk;
  const uint16_t* base = X + (size_t(bh) * N + size_t(i) * block) * HD;
  const int c8 = tid % CPR;
  const int rl = tid / CPR;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int row = rl; row < valid; row += RPP) {
    const uint4 u = *reinterpret_cast<const uint4*>(base + size_t(row) * HD + c8 * 8);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(w[e] << 16);
      acc[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rl][c8 * 8 + e] = acc[e];
  __syncthreads();
  if (tid < HD) {
    float s = 0.f;
    for (int rr = 0; rr < RPP; ++rr) s += red[rr][tid];
    P[size_t(blk) * HD + tid] = s / static_cast<float>(valid);
  }
}

template <int HD>
__global__ __launch_bounds__(256) void score_kernel(const float* __restrict__ Pq,
                                                    const float* __restrict__ Pk, int32_t nb,
                                                    float* __restrict__ S) {
  // A 32 x 32 tile of one head's scores per workgroup; thread (ti, tj) computes the
  // 2 x 2 block of rows 2ti, 2ti+1 and columns 2tj, 2tj+1, four dimensions per
  // step from 16-byte LDS reads (rows padded by 4 floats: 16-byte aligned, and
  // the 16 threads of a row group read 16 different bank groups).
  constexpr int LD = HD + 4;
  __shared__ __align__(16) float sq[32 * LD];
  __shared__ __align__(16) float sk[32 * LD];
  const int tid = threadIdx.x;
  const int j0 = blockIdx.x * 32;
  const int i0 = blockIdx.y * 32;
  const size_t bh = blockIdx.z;
  // Every thread's loads are issued before any is stored, so the workgroup
  // waits for one memory round trip, not one per load.
  constexpr int kPer = 32 * HD / 4 / 256;  // 16-byte loads per thread and operand
  static_assert(kPer * 256 == 32 * HD / 4, "the tile loads cover the threads evenly");
  f32x4 qv[kPer], kv[kPer];
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int x = tid + 256 * t;
    const int rr = x / (HD / 4);
    const int d = 4 * (x - rr * (HD / 4));
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    qv[t] = (i0 + rr < nb) ? *reinterpret_cast<const f32x4*>(Pq + (bh * nb + i0 + rr) * HD + d) : z;
    kv[t] = (j0 + rr < nb) ? *reinterpret_cast<const f32x4*>(Pk + (bh * nb + j0 + rr) * HD + d) : z;
  }
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int x = tid + 256 * t;
    const int rr = x / (HD / 4);
    const int d = 4 * (x - rr * (HD / 4));
    *reinterpret_cast<f32x4*>(sq + rr * LD + d) = qv[t];
    *reinterpret_cast<f32x4*>(sk + rr * LD + d) = kv[t];
  }
  __syncthreads();
  const int ti = tid >> 4;
  const int tj = tid & 15;
  float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
#pragma unroll 4
  for (int d = 0; d < HD; d += 4) {
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(sq + (2 * ti) * LD + d);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(sq + (2 * ti + 1) * LD + d);
    const f32x4 b0 = *reinterpret_cast<const f32x4*>(sk + (2 * tj) * LD + d);
    const f32x4 b1 = *reinterpret_cast<const f32x4*>(sk + (2 * tj + 1) * LD + d);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[0][0] = fmaf(a0[e], b0[e], acc[0][0]);
      acc[0][1] = fmaf(a0[e], b1[e], acc[0][1]);
      acc[1][0] = fmaf(a1[e], b0[e], acc[1][0]);
      acc[1][1] = fmaf(a1[e], b1[e], acc[1][1]);
    }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int i = i0 + 2 * ti + m;
    if (i >= nb) continue;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int j = j0 + 2 * tj + n;
      if (j < nb) S[(bh * nb + i) * nb + j] = acc[m][n];
    }
  }
}

// Order-preserving map of an fp32 score to uint32 (-0 folded onto +0).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f + 0.f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Set bits of a ballot mask below this lane.
__device__ __forceinline__ int popc_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// One wavefront per CSR row; CM = columns per lane (nb <= 64*CM).
template <int CM>
__global__ __launch_bounds__(256) void select_kernel(
    const float* __restrict__ S, const uint8_t* __restrict__ prior, int32_t prior_per_head,
    const int32_t* __restrict__ budgets, int32_t k_density, int32_t force_diag, int32_t nb,
    int32_t n_rows, const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
    int32_t* __restrict__ status) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  const int bh = r / nb;
  const int i = r - bh * nb;
  const uint8_t* pr =
      prior ? prior + (prior_per_head ? size_t(bh) * nb * nb : size_t(0)) + size_t(i) * nb
            : nullptr;
  const float* srow = S ? S + (size_t(bh) * nb + i) * nb : nullptr;
  // The row's prior bytes and scores, every load in flight at once: buffer loads
  // past the row (or from an absent prior or score matrix, a zero-size range)
  // read zero without touching memory.
  const __amdgpu_buffer_rsrc_t prr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(pr), static_cast<short>(0), pr ? nb : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(srow), static_cast<short>(0), srow ? nb * 4 : 0, 0x00020000);
  uint32_t pv[CM], sv[CM];
#pragma unroll
  for (int c = 0; c < CM; ++c) {
    const uint32_t j = static_cast<uint32_t>(min(lane + 64 * c, nb));
    pv[c] = __builtin_amdgcn_raw_buffer_load_b8(prr, j, 0, 0);
    sv[c] = __builtin_amdgcn_raw_buffer_load_b32(sr, j * 4u, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of their first use
  const int nnz = row_ptr[n_rows];
  const int start = row_ptr[r];
  const int cnt = row_ptr[r + 1] - start;
  // k_density < 0: the row keeps as many blocks as its CSR row has (the block
  // oracle at the density of a given CSR).
  const int ki = budgets ? min(max(budgets[i], 0), nb) : (k_density >= 0 ? k_density : min(max(cnt, 0), nb));

  uint64_t key[CM];
  bool insel[CM];
  bool chosen[CM];
  int nsel = 0;
#pragma unroll
  for (int c = 0; c < CM; ++c) {
    const int j = lane + 64 * c;
    const bool in = j < nb && (pv[c] != 0 || (force_diag && j == i));
    insel[c] = in;
    chosen[c] = false;
    key[c] = (j < nb && !in && srow)
                 ? ((uint64_t(ordered_bits(__uint_as_float(sv[c]))) << 32) | (0xffffffffu - uint32_t(j)))
                 : 0ull;
    nsel += __popcll(__ballot(in));
  }
  const int fill = max(0, ki - nsel);
  if (cnt != nsel + fill || start < 0 || start + cnt > nnz) {
    if (lane == 0) atomicAdd(status, 1);
    return;
  }
  // The `fill` largest keys (score, then lower column) among the candidates
  // (key != 0): a bitwise search finds H, the fill-th largest score word;
  // every candidate above H is taken, and of those equal to H the ones with
  // the lowest columns (column order is c-major, then lane) until `fill` are
  // taken.  Counts come from ballots, so the search costs the same for any fill.
  if (fill > 0) {
    uint32_t hi[CM];
    bool cand[CM];
    int n_cand = 0;
#pragma unroll
    for (int c = 0; c < CM; ++c) {
      cand[c] = key[c] != 0;
      hi[c] = static_cast<uint32_t>(key[c] >> 32);
      n_cand += __popcll(__ballot(cand[c]));
    }
    if (n_cand <= fill) {
#pragma unroll
      for (int c = 0; c < CM; ++c) chosen[c] = cand[c];
    } else {
      uint32_t H = 0;  // largest value with at least `fill` candidates at or above it
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t t = H | (1u << bit);
        int n = 0;
#pragma unroll
        for (int c = 0; c < CM; ++c) n += __popcll(__ballot(cand[c] && hi[c] >= t));
        if (n >= fill) H = t;
      }
      int above = 0;
#pragma unroll
      for (int c = 0; c < CM; ++c) above += __popcll(__ballot(cand[c] && hi[c] > H));
      const int need = fill - above;  // taken from the candidates equal to H
      int before = 0;                 // equal candidates in lower column blocks
#pragma unroll
      for (int c = 0; c < CM; ++c) {
        const bool eq = cand[c] && hi[c] == H;
        const uint64_t m = __ballot(eq);
        chosen[c] = (cand[c] && hi[c] > H) || (eq && before + popc_below(m) < need);
        before += __popcll(m);
      }
    }
  }
  int base = 0;
#pragma unroll
  for (int c = 0; c < CM; ++c) {
    const bool flag = insel[c] || chosen[c];
    const uint64_t m = __ballot(flag);
    if (flag) col_idx[start + base + popc_below(m)] = lane + 64 * c;
    base += __popcll(m);
  }
}

size_t round_up(size_t x) { return (x + 255) & ~size_t(255); }

struct MaskWs {
  size_t status, pq, pk, s, total;
};

MaskWs mask_ws_layout(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block) {
  const size_t nb = static_cast<size_t>(n_blocks(N, block));
  const size_t bhn = size_t(B) * H * nb;
  MaskWs w;
  w.status = 0;
  w.pq = kStatusBytes;
  w.pk = w.pq + round_up(bhn * D * 4);
  w.s = w.pk + round_up(bhn * D * 4);
  w.total = w.s + round_up(bhn * nb * 4);
  return w;
}

template <int CM>
void launch_select(const float* S, const uint8_t* prior, int32_t per_head, const int32_t* budgets,
                   int32_t kd, int32_t diag, int32_t nb, int32_t n_rows, const int32_t* row_ptr,
                   int32_t* col_idx, int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel<CM>, dim3((n_rows + 3) / 4), dim3(256), 0, s, S, prior,
                     per_head, budgets, kd, diag, nb, n_rows, row_ptr, col_idx, status);
}

}  // namespace
}  // namespace bsa

extern "C" BSA_API size_t bsa_build_mask_workspace_bytes(int32_t B, int32_t H, int32_t N,
                                                         int32_t D, int32_t block) {
  if (B < 1 || H < 1 || N < 1 || block < 1 || D < 1) return 0;
  return bsa::mask_ws_layout(B, H, N, D, block).total;
}

extern "C" BSA_API bsa_status bsa_build_mask(const void* q, const void* k, int32_t B, int32_t H,
                                             int32_t N, int32_t D, int32_t block, double density,
                                             const int32_t* budgets_dev, const uint8_t* prior_dev,
                                             int32_t prior_per_head, int32_t force_diag,
                                             const int32_t* row_ptr_dev, int32_t* col_idx_dev,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream) {
  using namespace bsa;
  if (!q || !k || !row_ptr_dev || !col_idx_dev || !workspace) return BSA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || density != density) return BSA_ERR_INVALID_ARG;
  if (!supported_shape(D, block)) return BSA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return BSA_ERR_INVALID_ARG;
  const int32_t nb = n_blocks(N, block);
  if (nb > kMaxBlocks) return BSA_ERR_UNSUPPORTED;
  const int64_t rows = int64_t(B) * H * nb;
  if (rows > INT32_MAX - 1) return BSA_ERR_UNSUPPORTED;
  const int32_t n_rows = static_cast<int32_t>(rows);
  const MaskWs w = mask_ws_layout(B, H, N, D, block);
  if (workspace_bytes < w.total) return BSA_ERR_CAPACITY;
  const int32_t kd = bsa_budget_from_density(nb, density);
  const bool need_scores = budgets_dev != nullptr || kd > 0;

  char* ws = static_cast<char*>(workspace);
  int32_t* status = reinterpret_cast<int32_t*>(ws + w.status);
  float* pq = reinterpret_cast<float*>(ws + w.pq);
  float* pk = reinterpret_cast<float*>(ws + w.pk);
  float* S = reinterpret_cast<float*>(ws + w.s);
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (need_scores) {
    // pool_kernel also clears the status word.
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    if (D == 64)
      hipLaunchKernelGGL(pool_kernel<64>, dim3(n_rows, 2), dim3(256), 0, s, qq, kk, N, nb, block,
                         pq, pk, status);
    else
      hipLaunchKernelGGL(pool_kernel<128>, dim3(n_rows, 2), dim3(256), 0, s, qq, kk, N, nb,
                         block, pq, pk, status);
    BSA_HIP_CHECK_LAUNCH();
    const dim3 g((nb + 31) / 32, (nb + 31) / 32, B * H);
    if (D == 64)
      hipLaunchKernelGGL(score_kernel<64>, g, dim3(256), 0, s, pq, pk, nb, S);
    else
      hipLaunchKernelGGL(score_kernel<128>, g, dim3(256), 0, s, pq, pk, nb, S);
    BSA_HIP_CHECK_LAUNCH();
  } else {
    hipLaunchKernelGGL(zero_status_kernel, dim3(1), dim3(1), 0, s, status);
    BSA_HIP_CHECK_LAUNCH();
  }
  const float* Sp = need_scores ? S : nullptr;
  const int32_t diag = force_diag ? 1 : 0;
  const int32_t ph = prior_per_head ? 1 : 0;
  if (nb <= 64)
    launch_select<1>(Sp, prior_dev, ph, budgets_dev, kd, diag, nb, n_rows, row_ptr_dev,
                     col_idx_dev, status, s);
  else if (nb <= 128)
    launch_select<2>(Sp, prior_dev, ph, budgets_dev, kd, diag, nb, n_rows, row_ptr_dev,
                     col_idx_dev, status, s);
  else if (nb <= 256)
    launch_select<4>(Sp, prior_dev, ph, budgets_dev, kd, diag, nb, n_rows, row_ptr_dev,
                     col_idx_dev, status, s);
  else if (nb <= 512)
    launch_select<8>(Sp, prior_dev, ph, budgets_dev, kd, diag, nb, n_rows, row_ptr_dev,
                     col_idx_dev, status, s);
  else
    launch_select<16>(Sp, prior_dev, ph, budgets_dev, kd, diag, nb, n_rows, row_ptr_dev,
                      col_idx_dev, status, s);
  BSA_HIP_CHECK_LAUNCH();
  return BSA_OK;
}

extern "C" BSA_API bsa_status bsa_select_by_mass(const float* mass_dev, int32_t n_rows, int32_t nb,
                                                 const int32_t* row_ptr_dev, int32_t* col_idx_dev,
                                                 int32_t* status_dev, void* stream) {
  using namespace bsa;
  if (!mass_dev || !row_ptr_dev || !col_idx_dev || !status_dev || n_rows < 1 || nb < 1)
    return BSA_ERR_INVALID_ARG;
  if (nb > kMaxBlocks) return BSA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(zero_status_kernel, dim3(1), dim3(1), 0, s, status_dev);
  BSA_HIP_CHECK_LAUNCH();
  // Rows are (head, block) pairs of nb rows each: prior none, no forced diagonal,
  // k from the row lengths.
  if (nb <= 64)
    launch_select<1>(mass_dev, nullptr, 0, nullptr, -1, 0, nb, n_rows, row_ptr_dev, col_idx_dev, status_dev, s);
  else if (nb <= 128)
    launch_select<2>(mass_dev, nullptr, 0, nullptr, -1, 0, nb, n_rows, row_ptr_dev, col_idx_dev, status_dev, s);
  else if (nb <= 256)
    launch_select<4>(mass_dev, nullptr, 0, nullptr, -1, 0, nb, n_rows, row_ptr_dev, col_idx_dev, status_dev, s);
  else if (nb <= 512)
    launch_select<8>(mass_dev, nullptr, 0, nullptr, -1, 0, nb, n_rows, row_ptr_dev, col_idx_dev, status_dev, s);
  else
    launch_select<16>(mass_dev, nullptr, 0, nullptr, -1, 0, nb, n_rows, row_ptr_dev, col_idx_dev, status_dev, s);
  BSA_HIP_CHECK_LAUNCH();
  return BSA_OK;
}

extern "C" BSA_API bsa_status bsa_build_mask_status(const void* workspace, void* stream,
                                                    int32_t* mismatched_rows) {
  if (!workspace || !mismatched_rows) return BSA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  if (hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess)
    return BSA_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return BSA_ERR_HIP;
  *mismatched_rows = v;
  return v == 0 ? BSA_OK : BSA_ERR_PLAN_MISMATCH;
}
