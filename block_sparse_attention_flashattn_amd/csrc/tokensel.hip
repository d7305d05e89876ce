// Token-level KV selection with tile-aligned query groups: the query grouping,
// the exact token mass per group and the top-k tokens of every group.
//
// Page "Can sparse attention close the quality gap in diffusion transformers"
// (MC-Sparse summary), section on token-level selection with tile-aligned query
// groups: KV tokens are chosen one by one per query group and gathered by index;
// the queries of one head are batched into groups of C similar queries, made by
// the median-split version of principal-direction divisive partitioning (each
// group projected on its principal direction and cut at the median,
// recursively); exact selection needs the attention scores (a two-pass kernel).
// Readings (the page leaves these steps open): the principal direction after
// kPowerIters power-iteration steps from u[d] = 1 + d/D; a group of g*C queries
// is cut into floor(g/2)*C and the rest, smallest projections (ties to the lower
// token) first, groups numbered depth first; a token's mass for a group is the
// dense attention probability summed over the group's queries.
#include "common.h"

namespace bsa {
namespace {

constexpr int kPowerIters = 8;
constexpr int kMaxTokens = 8192;  // tokens per head handled by the sorts (LDS)
constexpr int kMaxGroups = kMaxTokens / 64;  // group sizes are 64 or 128
constexpr int kThreads = 256;

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Order-preserving map of an fp32 value to uint32 (-0 folded onto +0).
__device__ __forceinline__ uint32_t ordered(float f) {
  const uint32_t u = __float_as_uint(f + 0.f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Ascending bitonic sort of keys[0, n) in LDS over stages of size up to max_size
// (n a power of two; with max_size < n every aligned run of max_size elements is
// sorted on its own).  All threads of the workgroup call it.
__device__ void bitonic(uint64_t* keys, int n, int max_size) {
  for (int size = 2; size <= max_size; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int t = threadIdx.x; t < n / 2; t += kThreads) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        // Runs alternate direction so that the next merge sees bitonic input; the
        // last merge sorts every run ascending.
        const bool up = size == max_size || (lo & size) == 0;
        const uint64_t a = keys[lo], b = keys[hi];
        if ((a > b) == up) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
    }
  __syncthreads();
}

// One workgroup per head.  `perm` (the output, [N]) holds the current order of the
// head's tokens; segments of whole groups are split level by level in place, so
// the final segments come out in depth-first order.
template <int HD>
__global__ __launch_bounds__(kThreads) void group_kernel(const uint16_t* __restrict__ Q, int32_t N,
                                                         int32_t C, int32_t* __restrict__ groups) {
  constexpr int RG = kThreads / HD;  // row groups of the dimension-parallel sums
  __shared__ uint64_t keys[kMaxTokens];
  __shared__ float red[RG][HD];
  __shared__ float mu[HD], v[HD];
  __shared__ int32_t seg_s[2 * kMaxGroups], seg_g[2 * kMaxGroups];  // list, then the next
  __shared__ int32_t nseg_sh;
  __shared__ float norm_sh;
  float* y = reinterpret_cast<float*>(keys);  // row dot products (reuses the key area)
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const uint16_t* q = Q + size_t(bh) * N * HD;
  int32_t* perm = groups + size_t(bh) * N;
  const int G = N / C;
  for (int r = tid; r < N; r += kThreads) perm[r] = r;
  if (tid == 0) {
    seg_s[0] = 0;
    seg_g[0] = G;
    nseg_sh = 1;
  }
  __syncthreads();
  for (;;) {
    const int nseg = nseg_sh;
    bool any = false;
    for (int s = 0; s < nseg; ++s) any |= seg_g[s] > 1;
    if (!any) break;
    __syncthreads();
    // New segment list written after the splits (at most doubling).
    int out_n = 0;
    for (int s = 0; s < nseg; ++s) {
      const int s0 = seg_s[s] * C, g = seg_g[s], n = g * C;
      if (g > 1) {
        const int32_t* idx = perm + s0;
        // mean
        {
          const int d = tid % HD, rg = tid / HD;
          float acc = 0.f;
          for (int j = rg; j < n; j += RG) acc += bf2f(q[size_t(idx[j]) * HD + d]);
          red[rg][d] = acc;
          __syncthreads();
          if (tid < HD) {
            float m = 0.f;
            for (int k = 0; k < RG; ++k) m += red[k][tid];
            mu[tid] = m / float(n);
            v[tid] = 1.f + float(tid) / float(HD);
          }
          __syncthreads();
          if (tid == 0) {
            float s2 = 0.f;
            for (int k = 0; k < HD; ++k) s2 += v[k] * v[k];
            norm_sh = sqrtf(s2);
          }
          __syncthreads();
          if (tid < HD) v[tid] /= norm_sh;
          __syncthreads();
        }
        for (int it = 0; it < kPowerIters; ++it) {
          for (int j = tid; j < n; j += kThreads) {
            const uint16_t* row = q + size_t(idx[j]) * HD;
            float a = 0.f;
            for (int k = 0; k < HD; ++k) a += (bf2f(row[k]) - mu[k]) * v[k];
            y[j] = a;
          }
          __syncthreads();
          {
            const int d = tid % HD, rg = tid / HD;
            float acc = 0.f;
            for (int j = rg; j < n; j += RG) acc += (bf2f(q[size_t(idx[j]) * HD + d]) - mu[d]) * y[j];
            red[rg][d] = acc;
          }
          __syncthreads();
          if (tid < HD) {
            float w = 0.f;
            for (int k = 0; k < RG; ++k) w += red[k][tid];
            red[0][tid] = w;
          }
          __syncthreads();
          if (tid == 0) {
            float s2 = 0.f;
            for (int k = 0; k < HD; ++k) s2 += red[0][k] * red[0][k];
            norm_sh = sqrtf(s2);
          }
          __syncthreads();
          const float nrm = norm_sh;
          if (nrm == 0.f) break;  // uniform: every thread reads the same value
          if (tid < HD) v[tid] = red[0][tid] / nrm;
          __syncthreads();
        }
        // projections -> sort keys (projection ascending, then token ascending)
        int npad = 1;
        while (npad < n) npad <<= 1;
        for (int j = tid; j < npad; j += kThreads) {
          if (j < n) {
            const uint16_t* row = q + size_t(idx[j]) * HD;
            float a = 0.f;
            for (int k = 0; k < HD; ++k) a += (bf2f(row[k]) - mu[k]) * v[k];
            keys[j] = (uint64_t(ordered(a)) << 32) | uint32_t(idx[j]);
          } else {
            keys[j] = ~0ull;
          }
        }
        bitonic(keys, npad, npad);
        for (int j = tid; j < n; j += kThreads) perm[s0 + j] = static_cast<int32_t>(keys[j] & 0xffffffffu);
        __syncthreads();
        const int gl = g / 2;
        if (tid == 0) {
          seg_s[nseg + out_n] = seg_s[s];
          seg_g[nseg + out_n] = gl;
          seg_s[nseg + out_n + 1] = seg_s[s] + gl;
          seg_g[nseg + out_n + 1] = g - gl;
        }
        out_n += 2;
      } else {
        if (tid == 0) {
          seg_s[nseg + out_n] = seg_s[s];
          seg_g[nseg + out_n] = 1;
        }
        out_n += 1;
      }
      __syncthreads();
    }
    // Move the new list to the front (out_n <= kMaxGroups <= kThreads).
    int a = 0, b = 0;
    if (tid < out_n) {
      a = seg_s[nseg + tid];
      b = seg_g[nseg + tid];
    }
    __syncthreads();
    if (tid < out_n) {
      seg_s[tid] = a;
      seg_g[tid] = b;
    }
    if (tid == 0) nseg_sh = out_n;
    __syncthreads();
  }
  // Every group's tokens ascending: bitonic stages up to C sort each aligned run.
  int npad = 1;
  while (npad < N) npad <<= 1;
  for (int j = tid; j < npad; j += kThreads) keys[j] = j < N ? uint64_t(uint32_t(perm[j])) : ~0ull;
  bitonic(keys, npad, C);
  for (int j = tid; j < N; j += kThreads) perm[j] = static_cast<int32_t>(keys[j] & 0xffffffffu);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           0x00020000);
}

__device__ __forceinline__ bf16x8 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Token mass of one group: one workgroup (four wavefronts) per (group, 128 keys);
// S = Q K^T with the group's queries as MFMA rows (gathered by index): lane
// (kl, hh) holds, for key kl of its 32, the queries 8(e/4) + 4hh + (e%4) of a
// 32-query slice, so summing over the group's queries is a sum over the lane's
// own values plus the other half-wavefront.
template <int CG, int HD>
__global__ __launch_bounds__(256) void token_mass_kernel(const uint16_t* __restrict__ Q,
                                                         const uint16_t* __restrict__ K,
                                                         const float* __restrict__ lse,
                                                         const int32_t* __restrict__ groups,
                                                         int32_t N, int32_t G, float sl2,
                                                         float* __restrict__ mass) {
  constexpr int QS = CG / 32;  // 32-query slices
  constexpr int NC = HD / 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kl = lane & 31, hh = lane >> 5;
  const int row = blockIdx.x;  // (head, group)
  const int bh = row / G;
  const int32_t* ids = groups + size_t(row) * CG;
  const size_t head = size_t(bh) * size_t(N) * HD;
  const uint32_t hbytes = static_cast<uint32_t>(N) * HD * 2u;
  const __amdgpu_buffer_rsrc_t qr = rsrc(Q + head, hbytes);
  const __amdgpu_buffer_rsrc_t kr = rsrc(K + head, hbytes);
  bf16x8 qf[QS][NC];
  float lq[QS][16];
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    const int t = ids[32 * s + kl];
    const bool ok = t >= 0 && t < N;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[s][c] = load16(qr, ok ? static_cast<uint32_t>(t * HD + 16 * c + 8 * hh) * 2u : hbytes);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int te = ids[32 * s + 8 * (e >> 2) + 4 * hh + (e & 3)];
      const float l = (te >= 0 && te < N) ? lse[size_t(bh) * N + te] : -INFINITY;
      lq[s][e] = (l > -INFINITY && l < INFINITY) ? l * 1.4426950408889634f : INFINITY;
    }
  }
  const int key = blockIdx.y * 128 + 32 * wave + kl;
  bf16x8 kf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    kf[c] = load16(kr, key < N ? static_cast<uint32_t>(key * HD + 16 * c + 8 * hh) * 2u : hbytes);
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    f32x16 sv = {};
#pragma unroll
    for (int c = 0; c < NC; ++c) sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[s][c], kf[c], sv, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc += __builtin_amdgcn_exp2f(fmaf(sv[e], sl2, -lq[s][e]));
  }
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc), __float_as_uint(acc), false, false);
  const float other = __uint_as_float(hh ? sw[0] : sw[1]);
  if (hh == 0 && key < N) mass[size_t(row) * N + key] = acc + other;
}

// Top-k tokens of one group's mass row (largest mass, ties to the lower token),
// ascending: one workgroup per row, two bitonic sorts in LDS.
__global__ __launch_bounds__(kThreads) void select_tokens_kernel(const float* __restrict__ mass,
                                                                 int32_t N, int32_t k,
                                                                 int32_t* __restrict__ tokens) {
  __shared__ uint64_t keys[kMaxTokens];
  const int row = blockIdx.x;
  const float* m = mass + size_t(row) * N;
  int npad = 1;
  while (npad < N) npad <<= 1;
  for (int j = threadIdx.x; j < npad; j += kThreads)
    keys[j] = j < N ? (uint64_t(~ordered(m[j])) << 32) | uint32_t(j) : ~0ull;
  bitonic(keys, npad, npad);
  int kpad = 1;
  while (kpad < k) kpad <<= 1;
  // The k chosen tokens, by index: each entry is rewritten by the thread that reads it.
  for (int j = threadIdx.x; j < kpad; j += kThreads)
    keys[j] = j < k ? (keys[j] & 0xffffffffu) : ~0ull;
  bitonic(keys, kpad, kpad);
  for (int j = threadIdx.x; j < k; j += kThreads) tokens[size_t(row) * k + j] = static_cast<int32_t>(keys[j]);
}

}  // namespace
}  // namespace bsa

extern "C" BSA_API bsa_status bsa_query_groups(const void* q, int32_t B, int32_t H, int32_t N,
                                               int32_t D, int32_t C, int32_t* groups_out,
                                               void* stream) {
  using namespace bsa;
  if (!q || !groups_out || B < 1 || H < 1 || N < 1 || C < 1) return BSA_ERR_INVALID_ARG;
  if (N % C != 0) return BSA_ERR_INVALID_ARG;
  if (N > kMaxTokens || (C != 64 && C != 128) || (D != 64 && D != 128)) return BSA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D == 64)
    hipLaunchKernelGGL(group_kernel<64>, dim3(B * H), dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(q), N, C, groups_out);
  else
    hipLaunchKernelGGL(group_kernel<128>, dim3(B * H), dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(q), N, C, groups_out);
  BSA_HIP_CHECK_LAUNCH();
  return BSA_OK;
}

extern "C" BSA_API bsa_status bsa_token_mass(const void* q, const void* k, const float* lse,
                                             const int32_t* groups, int32_t B, int32_t H,
                                             int32_t N, int32_t D, int32_t C, float scale,
                                             float* mass_out, void* stream) {
  using namespace bsa;
  if (!q || !k || !lse || !groups || !mass_out || B < 1 || H < 1 || N < 1) return BSA_ERR_INVALID_ARG;
  if (N % C != 0 || !(scale == scale)) return BSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k)) return BSA_ERR_INVALID_ARG;
  if ((C != 64 && C != 128) || (D != 64 && D != 128)) return BSA_ERR_UNSUPPORTED;
  if (int64_t(N) * D * 2 >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  const float sc = scale > 0.f ? scale : 1.f / sqrtf(static_cast<float>(D));
  const float sl2 = sc * 1.4426950408889634f;
  const int32_t G = N / C;
  const dim3 grid(B * H * G, (N + 127) / 128);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  if (C == 64 && D == 64)
    hipLaunchKernelGGL((token_mass_kernel<64, 64>), grid, dim3(256), 0, s, qq, kk, lse, groups, N, G, sl2, mass_out);
  else if (C == 64)
    hipLaunchKernelGGL((token_mass_kernel<64, 128>), grid, dim3(256), 0, s, qq, kk, lse, groups, N, G, sl2, mass_out);
  else if (D == 64)
    hipLaunchKernelGGL((token_mass_kernel<128, 64>), grid, dim3(256), 0, s, qq, kk, lse, groups, N, G, sl2, mass_out);
  else
    hipLaunchKernelGGL((token_mass_kernel<128, 128>), grid, dim3(256), 0, s, qq, kk, lse, groups, N, G, sl2, mass_out);
  BSA_HIP_CHECK_LAUNCH();
  return BSA_OK;
}

extern "C" BSA_API bsa_status bsa_select_tokens(const float* mass, int32_t n_rows, int32_t N,
                                                int32_t k, int32_t* tokens_out, void* stream) {
  using namespace bsa;
  if (!mass || !tokens_out || n_rows < 1 || N < 1 || k < 0 || k > N) return BSA_ERR_INVALID_ARG;
  if (N > kMaxTokens) return BSA_ERR_UNSUPPORTED;
  if (k == 0) return BSA_OK;
  hipLaunchKernelGGL(select_tokens_kernel, dim3(n_rows), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), mass, N, k, tokens_out);
  BSA_HIP_CHECK_LAUNCH();
  return BSA_OK;
}
