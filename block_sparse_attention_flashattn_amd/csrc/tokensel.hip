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
#include <algorithm>
#include <mutex>

#include "common.h"
#include "tile.h"

namespace bsa {
namespace {

constexpr int kPowerIters = 8;
constexpr int kMaxTokens = 8192;  // tokens per head (LDS key and token lists, register key arrays)
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

// ---------------------------------------------------------------------------
// Query groups, one launch pair per level of the split tree.  A segment of g
// groups (g > 1) at depth l becomes (s, g/2) and (s + g/2, g - g/2) at depth
// l + 1; its tokens occupy perm[s C, (s + g) C) of the head, so every segment of
// one depth can be split at the same time, each by its own workgroup.  The
// principal direction comes from the segment's scatter matrix
// M = sum (x - mu)(x - mu)^T (power iteration v <- M v / |M v|, the same map as
// X_c^T (X_c v) on the centred rows): large segments get M from fp32 partials of
// 512-token slices (many workgroups), combined in slice order with the
// parallel-variance update, small ones compute it in the splitting workgroup.

constexpr int kPart = 512;        // tokens per slice of a partial scatter matrix
constexpr int kDirectMax = 1024;  // segments up to this size compute M themselves

// The segments of one depth of the split tree that still hold more than one
// group, left to right (passed by value: a launch covers exactly these).
constexpr int kMaxNodes = 128;
struct NodeList {
  int32_t n;
  int32_t s[kMaxNodes];  // first group
  int32_t g[kMaxNodes];  // groups
};

// Scatter-matrix blocks of one thread: HD = 64, a 4x4 block (rows a0.., columns
// b0..); HD = 128, four 4x4 blocks (rows a0.., columns b0 + 32 k).
template <int HD>
struct ScatterBlock {
  static constexpr int NB = HD == 64 ? 1 : 4;
  f32x4 m[NB][4];
  int a0, b0;
  __device__ void init(int tid) {
    a0 = HD == 64 ? (tid >> 4) * 4 : (tid >> 3) * 4;
    b0 = HD == 64 ? (tid & 15) * 4 : (tid & 7) * 4;
#pragma unroll
    for (int k = 0; k < NB; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) m[k][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ int col(int k) const { return b0 + 32 * k; }
};

// LDS bytes slice_stats needs: the shifted rows of one 64-row batch as high and
// low bf16 halves (later the scatter matrix, in the same bytes), then per-thread
// partial row sums.
constexpr int stats_mat_bytes(int HD) { return 4 * 64 * HD > 4 * HD * HD ? 4 * 64 * HD : 4 * HD * HD; }
constexpr int stats_lds_bytes(int HD) { return stats_mat_bytes(HD) + kThreads * 8 * 4; }

// Mean and scatter matrix of the tokens ids[0, n) (LDS) of one head (rows of q):
// mu (LDS, HD floats) and this thread's blocks of M.  The rows are shifted by
// the first row x0 (fp32 differences of bf16 values are exact) and split into
// bf16 halves, v = hi + lo; S2 = sum (x - x0)(x - x0)^T accumulates on bf16
// MFMA (hi hi^T + hi lo^T + lo hi^T, fp32 accumulation: the dropped lo lo^T and
// the rounding of lo are ~2^-16 of each term), both operands read transposed
// from the staged rows (ds_read_b64_tr_b16).  S1 = sum (x - x0) in fp32,
// mu = x0 + S1 / n, M = S2 - S1 S1^T / n.  ws: stats_lds_bytes(HD) of LDS,
// 16-byte aligned; x0s: HD floats of LDS.  All threads of the workgroup call it.
template <int HD>
__device__ void slice_stats(const uint16_t* __restrict__ q, const int32_t* ids, int n, uint8_t* ws,
                            float* x0s, float* mu, ScatterBlock<HD>& sb) {
  constexpr int ROWB = HD * 2, CH = HD / 8, TILE = 64 * ROWB;
  constexpr int PT = 64 * CH / kThreads;  // 16-byte chunks per thread and batch
  constexpr int NTL = HD == 64 ? 1 : 4;   // 32x32 output tiles per wavefront
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, hh = lane >> 5;
  float* Mbuf = reinterpret_cast<float*>(ws);  // after the last batch
  float* s1p = reinterpret_cast<float*>(ws + stats_mat_bytes(HD));
  const uint32_t hiA = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((BSA_LDS uint8_t*)ws));
  const uint32_t loA = hiA + TILE;
  if (tid < HD) x0s[tid] = n > 0 ? bf2f(q[size_t(ids[0]) * HD + tid]) : 0.f;
  __syncthreads();
  // Thread tid's chunks always sit in column chunk tid % CH (kThreads % CH == 0).
  const int cc = tid % CH;
  float s1[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  f32x16 acc[NTL];
#pragma unroll
  for (int t = 0; t < NTL; ++t) acc[t] = f32x16{};
  const int ab = HD == 64 ? (wave >> 1) : wave;  // row block (a) of this wave's tiles
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  v4u pre[PT];
  auto fetch = [&](int j0) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int j = j0 + (tid + kThreads * u) / CH;
      pre[u] = j < n ? *reinterpret_cast<const v4u*>(q + size_t(ids[j]) * HD + 8 * cc)
                     : v4u{0u, 0u, 0u, 0u};
    }
  };
  // Operand [32 columns x 16 rows] of the staged tile at LDS address base,
  // columns 32 blk .. +31, rows 16 c2 .. +15 (the transposing read).
  auto opnd = [&](uint32_t base, int blk, int c2) -> bf16x8 {
    const int col = 32 * blk + tr_col;
    const v4s lo = lds_read_tr(base + swz<ROWB>(16 * c2 + tr_row, col >> 3) + (col & 7) * 2);
    const v4s hi = lds_read_tr(base + swz<ROWB>(16 * c2 + 8 + tr_row, col >> 3) + (col & 7) * 2);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  fetch(0);
  for (int j0 = 0; j0 < n; j0 += 64) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int r = (tid + kThreads * u) / CH;
      const bool ok = j0 + r < n;
      bf16x8 vh, vl;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t w = pre[u][x];
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          const int e = 2 * x + y;
          const float v = ok ? __uint_as_float(y ? (w & 0xffff0000u) : (w << 16)) - x0s[8 * cc + e]
                             : 0.f;
          s1[e] += v;
          const __bf16 h = static_cast<__bf16>(v);
          vh[e] = h;
          vl[e] = static_cast<__bf16>(v - static_cast<float>(h));
        }
      }
      *reinterpret_cast<BSA_LDS bf16x8*>(static_cast<uintptr_t>(hiA + swz<ROWB>(r, cc))) = vh;
      *reinterpret_cast<BSA_LDS bf16x8*>(static_cast<uintptr_t>(loA + swz<ROWB>(r, cc))) = vl;
    }
    __syncthreads();
    if (j0 + 64 < n) fetch(j0 + 64);
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) {
      const bf16x8 aH = opnd(hiA, ab, c2), aL = opnd(loA, ab, c2);
#pragma unroll
      for (int t = 0; t < NTL; ++t) {
        const int bb = HD == 64 ? (wave & 1) : t;
        const bf16x8 bH = opnd(hiA, bb, c2), bL = opnd(loA, bb, c2);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aH, bH, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aH, bL, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aL, bH, acc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // Tiles to LDS: lane (ql, hh) holds rows 32 ab + 8(e/4) + 4hh + e%4, column 32 bb + ql.
#pragma unroll
  for (int t = 0; t < NTL; ++t) {
    const int bb = HD == 64 ? (wave & 1) : t;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      Mbuf[(32 * ab + 8 * (e >> 2) + 4 * hh + (e & 3)) * HD + 32 * bb + ql] = acc[t][e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s1p[tid * 8 + e] = s1[e];
  __syncthreads();
  float S1 = 0.f;
  if (tid < HD) {
    for (int t = tid / 8; t < kThreads; t += CH) S1 += s1p[t * 8 + (tid & 7)];
    mu[tid] = n > 0 ? x0s[tid] + S1 / float(n) : 0.f;
  }
  __syncthreads();
  if (tid < HD) s1p[tid] = S1;
  __syncthreads();
  const float inv = n > 0 ? 1.f / float(n) : 0.f;
  sb.init(tid);
  const f32x4 sa = *reinterpret_cast<const f32x4*>(s1p + sb.a0);
#pragma unroll
  for (int k = 0; k < ScatterBlock<HD>::NB; ++k) {
    const f32x4 sbk = *reinterpret_cast<const f32x4*>(s1p + sb.col(k));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sb.m[k][i] = *reinterpret_cast<const f32x4*>(Mbuf + (sb.a0 + i) * HD + sb.col(k)) -
                   (sa[i] * inv) * sbk;
  }
  __syncthreads();
}

// Identity order of every head's tokens.
__global__ __launch_bounds__(kThreads) void perm_init_kernel(int32_t N, int32_t* __restrict__ perm) {
  const int bh = blockIdx.y;
  for (int r = blockIdx.x * kThreads + threadIdx.x; r < N; r += gridDim.x * kThreads)
    perm[size_t(bh) * N + r] = r;
}

// Partial (n, mu, M) of slice p of the segment of node b of the depth's list:
// grid (nodes * P, B*H); floats per partial 1 + HD + HD^2.
template <int HD>
__global__ __launch_bounds__(kThreads) void stats_kernel(const uint16_t* __restrict__ Q, int32_t N,
                                                         int32_t C, NodeList nodes, int32_t P,
                                                         const int32_t* __restrict__ perm,
                                                         float* __restrict__ part) {
  extern __shared__ __align__(16) uint8_t sws[];  // stats_lds_bytes(HD), then the token list
  __shared__ float mu[HD], x0s[HD];
  int32_t* ids = reinterpret_cast<int32_t*>(sws + stats_lds_bytes(HD));
  const int bh = blockIdx.y;
  const int b = blockIdx.x / P, p = blockIdx.x - b * P;
  const int s = nodes.s[b], g = nodes.g[b];
  const int n = g * C;
  const int L = (n + P - 1) / P;
  const int lo = min(p * L, n), hi = min(lo + L, n);
  const uint16_t* q = Q + size_t(bh) * N * HD;
  const int32_t* idx = perm + size_t(bh) * N + size_t(s) * C + lo;
  for (int j = threadIdx.x; j < hi - lo; j += kThreads) ids[j] = idx[j];
  __syncthreads();
  ScatterBlock<HD> sb;
  slice_stats<HD>(q, ids, hi - lo, sws, x0s, mu, sb);
  constexpr int F = 1 + HD + HD * HD;
  float* out = part + ((size_t(bh) * nodes.n + b) * P + p) * F;
  const int tid = threadIdx.x;
  if (tid == 0) out[0] = float(hi - lo);
  if (tid < HD) out[1 + tid] = mu[tid];
  float* M = out + 1 + HD;
#pragma unroll
  for (int k = 0; k < ScatterBlock<HD>::NB; ++k)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) M[(sb.a0 + i) * HD + sb.col(k) + j] = sb.m[k][i][j];
}

// Sums over lane groups without LDS, every lane of the group receiving the sum:
// DPP exchanges inside a 16-lane row (lane ^ 1, lane ^ 2, mirror within 8,
// mirror within 16), then v_permlane16_swap / v_permlane32_swap across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xf,
                                                    0xf, false));
}
__device__ __forceinline__ float row_sum8(float v) {
  v += dpp_f32<0xb1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f32<0x4e>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  return v;
}
__device__ __forceinline__ float row_sum16(float v) {
  v = row_sum8(v);
  v += dpp_f32<0x140>(v);  // row_mirror
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v += __uint_as_float((threadIdx.x & 16) ? s16[0] : s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v += __uint_as_float((threadIdx.x & 32) ? s32[0] : s32[1]);
  return v;
}

// w = scale M v for a scatter matrix held in ScatterBlocks (M symmetric, each thread
// its blocks): per-thread partial rows, summed over the lanes that share a row
// block (16 consecutive lanes at HD = 64, 8 at HD = 128), into w (LDS, HD floats).
template <int HD>
__device__ void scatter_matvec(const ScatterBlock<HD>& sb, const float* v, float* w, float scale) {
  f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < ScatterBlock<HD>::NB; ++k) {
    const f32x4 vb = *reinterpret_cast<const f32x4*>(v + sb.col(k));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      part[i] += sb.m[k][i][0] * vb[0] + sb.m[k][i][1] * vb[1] + sb.m[k][i][2] * vb[2] +
                 sb.m[k][i][3] * vb[3];
  }
  constexpr int span = HD == 64 ? 16 : 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) part[i] = (span == 16 ? row_sum16(part[i]) : row_sum8(part[i])) * scale;
  if ((threadIdx.x & (span - 1)) == 0) *reinterpret_cast<f32x4*>(w + sb.a0) = part;
}

// Euclidean norm of x[0, HD) (LDS), computed by wavefront 0 and left in *out.
template <int HD>
__device__ void norm_w0(const float* x, float* out) {
  if (threadIdx.x < 64) {
    float s2 = 0.f;
#pragma unroll
    for (int h = 0; h < HD / 64; ++h) s2 += x[64 * h + threadIdx.x] * x[64 * h + threadIdx.x];
    s2 = wave_sum(s2);
    if (threadIdx.x == 0) *out = sqrtf(s2);
  }
}

// Exclusive prefix sum over the workgroup's threads (one value each, thread
// order): a shuffle scan in each wavefront, then the wavefront totals through
// tmp (kThreads / 64 ints of LDS).  All threads call it.
__device__ int block_excl_scan(int x, int32_t* tmp) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) tmp[w] = incl;
  __syncthreads();
  int base = 0;
  for (int k = 0; k < w; ++k) base += tmp[k];
  __syncthreads();  // tmp is free for the next call
  return base + incl - x;
}

// Split of the segment of node b of the depth's list (grid (nodes, B*H)): its
// scatter matrix (from the P partials in slice order, or computed here when
// P == 1; either way held in registers, ScatterBlock), the principal direction,
// the projections, and the segment's tokens rewritten so that the floor(g/2) C
// smallest (projection, token) keys come first (the left child), each side in
// its previous order.  Dynamic LDS: the keys of the level's largest segment
// (and the row staging), then its token list.
template <int HD, bool WIDE>
__global__ __launch_bounds__(kThreads) void split_kernel(const uint16_t* __restrict__ Q, int32_t N,
                                                         int32_t C, NodeList nodes, int32_t P,
                                                         int32_t key_words,
                                                         const float* __restrict__ part,
                                                         int32_t* __restrict__ perm) {
  extern __shared__ __align__(16) uint64_t keys[];  // 16-byte aligned: slice_stats stages rows here
  __shared__ __align__(16) float red[kThreads / HD][HD];
  __shared__ float x0s[HD];
  __shared__ __align__(16) float mu[HD];
  __shared__ __align__(16) float v[HD];
  __shared__ __align__(16) float dl[HD];
  __shared__ float norm_sh, nacc_sh;
  __shared__ int32_t scan_sh[kThreads], sel_sh[3];
  __shared__ uint64_t pivot_sh;
  const int tid = threadIdx.x;
  const int bh = blockIdx.y, b = blockIdx.x;
  const int s = nodes.s[b], g = nodes.g[b];
  const int n = g * C, s0 = s * C;
  const uint16_t* q = Q + size_t(bh) * N * HD;
  int32_t* idx = perm + size_t(bh) * N + s0;
  // The segment's tokens, after the key (and staging) area.
  int32_t* ids = reinterpret_cast<int32_t*>(keys) + 2 * key_words;
  for (int j = tid; j < n; j += kThreads) ids[j] = idx[j];
  __syncthreads();
  constexpr int F = 1 + HD + HD * HD;
  ScatterBlock<HD> sb;
  if (P <= 1) {
    slice_stats<HD>(q, ids, n, reinterpret_cast<uint8_t*>(keys), x0s, mu, sb);
  } else {
    // (n, mu, M) <- (n, mu, M) + partial: delta = mu_p - mu, M += M_p +
    // n n_p / (n + n_p) delta delta^T, mu += delta n_p / (n + n_p).
    sb.init(tid);
    const float* pp = part + ((size_t(bh) * nodes.n + b) * P) * F;
    if (tid < HD) mu[tid] = 0.f;
    if (tid == 0) nacc_sh = 0.f;
    __syncthreads();
    for (int p = 0; p < P; ++p) {
      const float* src = pp + size_t(p) * F;
      const float na = nacc_sh, np = src[0];
      const float nt = na + np;
      if (np > 0.f) {  // uniform
        if (tid < HD) dl[tid] = src[1 + tid] - mu[tid];
        __syncthreads();
        const float f = na * np / nt;
        const f32x4 da = *reinterpret_cast<const f32x4*>(dl + sb.a0);
#pragma unroll
        for (int k = 0; k < ScatterBlock<HD>::NB; ++k) {
          const f32x4 db = *reinterpret_cast<const f32x4*>(dl + sb.col(k));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 mp =
                *reinterpret_cast<const f32x4*>(src + 1 + HD + (sb.a0 + i) * HD + sb.col(k));
            sb.m[k][i] += mp + (f * da[i]) * db;
          }
        }
        __syncthreads();
        if (tid < HD) mu[tid] += dl[tid] * (np / nt);
        if (tid == 0) nacc_sh = nt;
      }
      __syncthreads();
    }
  }
  __syncthreads();
  // Power iteration from u[d] = 1 + d / HD on M / trace(M) (spectral norm at
  // most 1: no overflow, and eight steps shrink v by at most (HD)^-8), one
  // barrier per step; the direction is normalised once at the end.  trace(M) = 0
  // (every row equal) or M u = 0 keeps u.
  {
    float dsum = 0.f;
    bool diag = false;
#pragma unroll
    for (int k = 0; k < ScatterBlock<HD>::NB; ++k)
      if (sb.a0 == sb.col(k)) {
        dsum = sb.m[k][0][0] + sb.m[k][1][1] + sb.m[k][2][2] + sb.m[k][3][3];
        diag = true;
      }
    if (diag) dl[sb.a0 / 4] = dsum;  // one thread per 4-row block
  }
  float* w = &red[0][0];  // two HD-float buffers, used in turn
  if (tid < HD) w[tid] = 1.f + float(tid) / float(HD);
  __syncthreads();
  float tr = 0.f;
#pragma unroll 8
  for (int i = 0; i < HD / 4; ++i) tr += dl[i];
  const float inv_tr = tr > 1e-30f ? 1.f / tr : 0.f;
  int cur = 0;
  if (inv_tr > 0.f) {
#pragma unroll 1
    for (int it = 0; it < kPowerIters; ++it) {
      scatter_matvec<HD>(sb, w + cur * HD, w + (cur ^ 1) * HD, inv_tr);
      cur ^= 1;
      __syncthreads();
    }
  }
  norm_w0<HD>(w + cur * HD, &norm_sh);
  __syncthreads();
  if (tid < HD) v[tid] = norm_sh > 0.f ? w[cur * HD + tid] / norm_sh : 1.f + float(tid) / float(HD);
  __syncthreads();
  // Projections -> keys (projection ascending, then token ascending).  WIDE
  // (segments split from slice partials, few workgroups): tokens strided over
  // the threads, two rows in flight per thread; otherwise (many workgroups,
  // where occupancy matters) each thread's own keys one row at a time.
  // Afterwards thread tid owns the contiguous keys [tid per, (tid + 1) per).
  auto proj = [&](const v4u* x) {
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < HD / 8; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 8 * c + 2 * e;
        a += (__uint_as_float(x[c][e] << 16) - mu[d]) * v[d];
        a += (__uint_as_float(x[c][e] & 0xffff0000u) - mu[d + 1]) * v[d + 1];
      }
    return a;
  };
  const int per = (n + kThreads - 1) / kThreads;
  const int jlo = min(tid * per, n), jhi = min(jlo + per, n);
  if constexpr (WIDE) {
    for (int j = tid; j < n; j += 2 * kThreads) {
      const int j2 = j + kThreads;
      const int t = ids[j], t2 = j2 < n ? ids[j2] : t;
      v4u x[HD / 8], x2[HD / 8];
#pragma unroll
      for (int c = 0; c < HD / 8; ++c) {
        x[c] = *reinterpret_cast<const v4u*>(q + size_t(t) * HD + 8 * c);
        x2[c] = *reinterpret_cast<const v4u*>(q + size_t(t2) * HD + 8 * c);
      }
      keys[j] = (uint64_t(ordered(proj(x))) << 32) | uint32_t(t);
      if (j2 < n) keys[j2] = (uint64_t(ordered(proj(x2))) << 32) | uint32_t(t2);
    }
    __syncthreads();
  } else {
    // Eight lanes per row (lane part c8 holds dimensions [HD/8 c8, +HD/8)), four
    // rows per lane octet in flight; the octet's partial dots meet by DPP.
    constexpr int DP = HD / 8, U = 4;
    const int c8 = tid & 7, slot = tid >> 3;
    float mv[DP], vv[DP];
#pragma unroll
    for (int e = 0; e < DP; ++e) {
      mv[e] = mu[DP * c8 + e];
      vv[e] = v[DP * c8 + e];
    }
    for (int j0 = slot; j0 < n; j0 += U * (kThreads / 8)) {
      v4u x[U][DP / 8];
      int t[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * (kThreads / 8);
        t[u] = ids[j < n ? j : j0];
#pragma unroll
        for (int c = 0; c < DP / 8; ++c)
          x[u][c] = *reinterpret_cast<const v4u*>(q + size_t(t[u]) * HD + DP * c8 + 8 * c);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < DP / 8; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int d = 8 * c + 2 * e;
            a += (__uint_as_float(x[u][c][e] << 16) - mv[d]) * vv[d];
            a += (__uint_as_float(x[u][c][e] & 0xffff0000u) - mv[d + 1]) * vv[d + 1];
          }
        a = row_sum8(a);
        const int j = j0 + u * (kThreads / 8);
        if (c8 == 0 && j < n) keys[j] = (uint64_t(ordered(a)) << 32) | uint32_t(t[u]);
      }
    }
    __syncthreads();
  }
  // The left child is the k = floor(g/2) C smallest keys (keys are distinct: the
  // token is part of them).  Radix select of the k-th smallest key, 8 bits at a
  // time from the top, then a stable partition: smaller keys to the front in
  // their current order, the rest after them.
  int32_t* hist = reinterpret_cast<int32_t*>(&red[0][0]);  // 256 bins (red holds >= 256 floats)
  uint64_t prefix = 0, mask = 0;
  int want = (g >> 1) * C;
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int j = jlo; j < jhi; ++j)
      if ((keys[j] & mask) == prefix) atomicAdd(&hist[(keys[j] >> shift) & 255], 1);
    __syncthreads();
    const int cnt = hist[tid];
    const int excl = block_excl_scan(cnt, scan_sh);
    if (excl <= want && want < excl + cnt) {
      sel_sh[0] = tid;
      sel_sh[1] = want - excl;
      sel_sh[2] = cnt;
    }
    __syncthreads();
    prefix |= uint64_t(sel_sh[0]) << shift;
    mask |= uint64_t(255) << shift;
    want = sel_sh[1];
    const int left = sel_sh[2];
    __syncthreads();
    if (left == 1) break;  // uniform: one candidate key has this prefix
  }
  // The pivot: the one key with the selected prefix (the k-th smallest).
  for (int j = jlo; j < jhi; ++j)
    if ((keys[j] & mask) == prefix) pivot_sh = keys[j];
  __syncthreads();
  const uint64_t pivot = pivot_sh;
  int nl = 0;
  for (int j = jlo; j < jhi; ++j) nl += keys[j] < pivot ? 1 : 0;
  const int kleft = (g >> 1) * C;
  int pl = block_excl_scan(nl, scan_sh);  // left slots before this thread
  int pr = kleft + (jlo - pl);             // right slots before this thread
  for (int j = jlo; j < jhi; ++j) {
    const uint64_t key = keys[j];
    const int32_t t = static_cast<int32_t>(key & 0xffffffffu);
    if (key < pivot)
      idx[pl++] = t;
    else
      idx[pr++] = t;
  }
}

// 64-bit words of split_kernel's key (and row staging) area for segments of up
// to nmax tokens; the segment's token list follows it (nmax int32).
inline int split_key_words(int nmax, int D) {
  return std::max((nmax + 1) & ~1, stats_lds_bytes(D) / 8);
}
inline size_t split_lds_bytes(int nmax, int D) {
  return size_t(split_key_words(nmax, D)) * 8 + size_t(nmax) * 4;
}

// Every group's tokens ascending: grid (G, B*H).
__global__ __launch_bounds__(kThreads) void group_sort_kernel(int32_t N, int32_t C,
                                                              int32_t* __restrict__ perm) {
  __shared__ uint64_t keys[128];
  int32_t* grp = perm + size_t(blockIdx.y) * N + size_t(blockIdx.x) * C;
  for (int j = threadIdx.x; j < C; j += kThreads) keys[j] = uint32_t(grp[j]);
  bitonic(keys, C, C);
  for (int j = threadIdx.x; j < C; j += kThreads) grp[j] = static_cast<int32_t>(keys[j]);
}

// Levels of the split tree that have a segment of more than one group, the
// slice count of each (1: the split workgroup computes M itself), and the
// partial floats the largest level needs.
struct GroupLevels {
  int depth = 0;
  int P[32] = {};
  size_t part_floats = 0;
};

inline GroupLevels group_levels(int32_t BH, int32_t N, int32_t D, int32_t C) {
  GroupLevels L;
  const int G = N / C;
  for (int l = 0; l < 31; ++l) {
    const int gmax = (G + (1 << l) - 1) >> l;  // the largest segment at depth l
    if (gmax <= 1) break;
    const int nmax = gmax * C;
    L.P[l] = nmax > kDirectMax ? (nmax + kPart - 1) / kPart : 1;
    if (L.P[l] > 1)
      L.part_floats = std::max(L.part_floats, size_t(BH) * (size_t(1) << l) * size_t(L.P[l]) *
                                                  size_t(1 + D + D * D));
    L.depth = l + 1;
  }
  return L;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           0x00020000);
}

__device__ __forceinline__ bf16x8 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Token mass of one group: one workgroup (four wavefronts) per (group, slice of
// the key tiles of 128 keys);
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
  // Each lane loads its own query's row fragments and LSE (one index load and
  // one LSE load per slice, all in flight together); the LSEs of the queries a
  // lane's accumulator rows hold then come from the lanes that loaded them.
  bf16x8 qf[QS][NC];
  float lq[QS][16];
  float lown[QS];
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    const int t = ids[32 * s + kl];
    const bool ok = t >= 0 && t < N;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[s][c] = load16(qr, ok ? static_cast<uint32_t>(t * HD + 16 * c + 8 * hh) * 2u : hbytes);
    const float l = ok ? lse[size_t(bh) * N + t] : -INFINITY;
    lown[s] = (l > -INFINITY && l < INFINITY) ? l * 1.4426950408889634f : INFINITY;
  }
#pragma unroll
  for (int s = 0; s < QS; ++s)
#pragma unroll
    for (int e = 0; e < 16; ++e) lq[s][e] = __shfl(lown[s], 8 * (e >> 2) + 4 * hh + (e & 3));
  // Key tiles blockIdx.y, blockIdx.y + gridDim.y, ...: the group's query
  // fragments and LSEs stay in registers; the next tile's K rows are in flight
  // while this one is used.
  const int n_tiles = (N + 127) / 128;
  auto fetch = [&](int kt, bf16x8 (&kf)[NC]) {
    const int key = kt * 128 + 32 * wave + kl;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      kf[c] = load16(kr, key < N ? static_cast<uint32_t>(key * HD + 16 * c + 8 * hh) * 2u : hbytes);
  };
  // No branch around the prefetch or the store: tiles past the end read zeros
  // (out-of-range offsets) and the dropped lanes store past the row's end, so the
  // waits for this tile's K never also wait for the next tile's loads.
  const __amdgpu_buffer_rsrc_t mrow =
      rsrc(mass + size_t(row) * N, static_cast<uint32_t>(N) * 4u);
  bf16x8 kf[NC], kn[NC];
  int kt = blockIdx.y;
  fetch(kt, kf);
  for (; kt < n_tiles; kt += gridDim.y) {
    fetch(kt + gridDim.y, kn);
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      f32x16 sv = {};
#pragma unroll
      for (int c = 0; c < NC; ++c)
        sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[s][c], kf[c], sv, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 16; ++e) acc += __builtin_amdgcn_exp2f(fmaf(sv[e], sl2, -lq[s][e]));
    }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc), __float_as_uint(acc),
                                                     false, false);
    const float other = __uint_as_float(hh ? sw[0] : sw[1]);
    const int key = kt * 128 + 32 * wave + kl;
    __builtin_amdgcn_raw_buffer_store_b32(
        __float_as_uint(acc + other), mrow,
        static_cast<uint32_t>(hh == 0 && key < N ? key : N) * 4u, 0, 0);
#pragma unroll
    for (int c = 0; c < NC; ++c) kf[c] = kn[c];
  }
}

// Top-k tokens of one group's mass row (largest mass, ties to the lower token),
// ascending: one workgroup per row.  Keys (~ordered(mass), token) are distinct and
// ascend with the wanted order; thread tid holds the keys of tokens
// [tid per, (tid + 1) per) in registers.  A radix select (11 bits at a time from
// the top) finds the k-th smallest key; the keys below it are the chosen tokens,
// written in token order by a workgroup scan of the per-thread counts.
constexpr int kSelPer = kMaxTokens / kThreads;  // keys per thread at most

__global__ __launch_bounds__(kThreads) void select_tokens_kernel(const float* __restrict__ mass,
                                                                 int32_t N, int32_t k,
                                                                 int32_t* __restrict__ tokens) {
  constexpr int kBits = 11, kBins = 1 << kBits, kPerT = kBins / kThreads;
  __shared__ int32_t hist[kBins], scan_sh[kThreads / 64], sel_sh[3];
  __shared__ uint64_t pivot_sh;
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const float* m = mass + size_t(row) * N;
  int32_t* out = tokens + size_t(row) * k;
  const int per = (N + kThreads - 1) / kThreads;
  const int jlo = min(tid * per, N), jhi = min(jlo + per, N);
  // The high word of each key in registers; the low word is the token, jlo + u.
  // Buffer loads (an out-of-range offset reads zero without touching memory) so
  // that all of a thread's loads are in flight together.
  const __amdgpu_buffer_rsrc_t mr = rsrc(m, static_cast<uint32_t>(N) * 4u);
  uint32_t kh[kSelPer];
#pragma unroll
  for (int u = 0; u < kSelPer; ++u) {
    const int j = jlo + u;
    kh[u] = __builtin_amdgcn_raw_buffer_load_b32(
        mr, static_cast<uint32_t>(u < per && j < jhi ? j : N) * 4u, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of their first use
#pragma unroll
  for (int u = 0; u < kSelPer; ++u)
    kh[u] = u < per && jlo + u < jhi ? ~ordered(__uint_as_float(kh[u])) : ~0u;
  auto valid = [&](int u) { return u < per && jlo + u < jhi; };
  auto keyof = [&](int u) { return (uint64_t(kh[u]) << 32) | uint32_t(jlo + u); };
  uint64_t pivot = ~0ull;  // k == N: every key is below no pivot; take them all
  if (k < N) {
    // 11-bit digits from the top (bits [53, 64), [42, 53), ...): the first digit
    // holds the mass's exponent and three mantissa bits, which spreads the LDS
    // histogram's atomics over many more bins than a byte of exponent would.
    uint64_t prefix = 0, mask = 0;
    int want = k;
    for (int top = 64; top > 0; top -= kBits) {
      const int shift = top > kBits ? top - kBits : 0;
      const uint32_t dmask = (1u << (top - shift)) - 1u;
#pragma unroll
      for (int i = 0; i < kPerT; ++i) hist[kPerT * tid + i] = 0;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kSelPer; ++u)
        if (valid(u) && (keyof(u) & mask) == prefix)
          atomicAdd(&hist[uint32_t(keyof(u) >> shift) & dmask], 1);
      __syncthreads();
      int c[kPerT], cnt = 0;
#pragma unroll
      for (int i = 0; i < kPerT; ++i) {
        c[i] = hist[kPerT * tid + i];
        cnt += c[i];
      }
      int excl = block_excl_scan(cnt, scan_sh);
      if (excl <= want && want < excl + cnt) {
#pragma unroll
        for (int i = 0; i < kPerT; ++i) {
          if (excl <= want && want < excl + c[i]) {
            sel_sh[0] = kPerT * tid + i;
            sel_sh[1] = want - excl;
            sel_sh[2] = c[i];
          }
          excl += c[i];
        }
      }
      __syncthreads();
      prefix |= uint64_t(sel_sh[0]) << shift;
      mask |= uint64_t(dmask) << shift;
      want = sel_sh[1];
      const int left = sel_sh[2];
      __syncthreads();
      if (left == 1) break;  // uniform
    }
#pragma unroll
    for (int u = 0; u < kSelPer; ++u)
      if (valid(u) && (keyof(u) & mask) == prefix) pivot_sh = keyof(u);
    __syncthreads();
    pivot = pivot_sh;
  }
  int nl = 0;
#pragma unroll
  for (int u = 0; u < kSelPer; ++u) nl += (valid(u) && (k >= N || keyof(u) < pivot)) ? 1 : 0;
  int pos = block_excl_scan(nl, scan_sh);
#pragma unroll
  for (int u = 0; u < kSelPer; ++u)
    if (valid(u) && (k >= N || keyof(u) < pivot)) out[pos++] = jlo + u;
}

}  // namespace
}  // namespace bsa

extern "C" BSA_API size_t bsa_query_groups_workspace_bytes(int32_t B, int32_t H, int32_t N,
                                                          int32_t D, int32_t C) {
  using namespace bsa;
  if (B < 1 || H < 1 || N < 1 || (C != 64 && C != 128) || (D != 64 && D != 128) || N % C)
    return 0;
  return std::max<size_t>(256, group_levels(B * H, N, D, C).part_floats * sizeof(float));
}

extern "C" BSA_API bsa_status bsa_query_groups(const void* q, int32_t B, int32_t H, int32_t N,
                                               int32_t D, int32_t C, int32_t* groups_out,
                                               void* workspace, size_t workspace_bytes,
                                               void* stream) {
  using namespace bsa;
  if (!q || !groups_out || !workspace || B < 1 || H < 1 || N < 1 || C < 1)
    return BSA_ERR_INVALID_ARG;
  if (N % C != 0 || !aligned16(q) || !aligned16(workspace)) return BSA_ERR_INVALID_ARG;
  if (N > kMaxTokens || (C != 64 && C != 128) || (D != 64 && D != 128)) return BSA_ERR_UNSUPPORTED;
  if (int64_t(B) * H > 65535) return BSA_ERR_UNSUPPORTED;
  if (workspace_bytes < bsa_query_groups_workspace_bytes(B, H, N, D, C)) return BSA_ERR_CAPACITY;
  const GroupLevels L = group_levels(B * H, N, D, C);
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    const int big = int(split_lds_bytes(kMaxTokens, 128));
    for (const void* f : {reinterpret_cast<const void*>(&split_kernel<64, false>),
                          reinterpret_cast<const void*>(&split_kernel<64, true>),
                          reinterpret_cast<const void*>(&split_kernel<128, false>),
                          reinterpret_cast<const void*>(&split_kernel<128, true>)})
      if (attr == hipSuccess)
        attr = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, big);
    for (const void* f : {reinterpret_cast<const void*>(&stats_kernel<64>),
                          reinterpret_cast<const void*>(&stats_kernel<128>)})
      if (attr == hipSuccess)
        attr = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   stats_lds_bytes(128) + kPart * 4);
  });
  if (attr != hipSuccess) return BSA_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  float* part = static_cast<float*>(workspace);
  const uint32_t bh = static_cast<uint32_t>(B * H);
  hipLaunchKernelGGL(perm_init_kernel, dim3((N + kThreads - 1) / kThreads, bh), dim3(kThreads), 0,
                     s, N, groups_out);
  BSA_HIP_CHECK_LAUNCH();
  // The split tree level by level: only the segments that still hold more than
  // one group are launched (the last level of t2i has 2 of 64 possible nodes).
  NodeList cur{};
  cur.n = 0;
  if (N / C > 1) {
    cur.n = 1;
    cur.s[0] = 0;
    cur.g[0] = N / C;
  }
  for (int l = 0; cur.n > 0; ++l) {
    const uint32_t nodes = static_cast<uint32_t>(cur.n);
    int gmax = 0;
    for (int x = 0; x < cur.n; ++x) gmax = std::max(gmax, cur.g[x]);
    const int P = L.P[l];
    if (P > 1) {
      if (D == 64)
        hipLaunchKernelGGL(stats_kernel<64>, dim3(nodes * P, bh), dim3(kThreads),
                           stats_lds_bytes(64) + kPart * 4, s, qq, N, C, cur, P, groups_out, part);
      else
        hipLaunchKernelGGL(stats_kernel<128>, dim3(nodes * P, bh), dim3(kThreads),
                           stats_lds_bytes(128) + kPart * 4, s, qq, N, C, cur, P, groups_out, part);
      BSA_HIP_CHECK_LAUNCH();
    }
    const size_t lds = split_lds_bytes(gmax * C, D);
    const int kw = split_key_words(gmax * C, D);
    auto* split = D == 64 ? (P > 1 ? split_kernel<64, true> : split_kernel<64, false>)
                          : (P > 1 ? split_kernel<128, true> : split_kernel<128, false>);
    hipLaunchKernelGGL(split, dim3(nodes, bh), dim3(kThreads), lds, s, qq, N, C, cur, P, kw, part,
                       groups_out);
    BSA_HIP_CHECK_LAUNCH();
    NodeList nxt{};
    nxt.n = 0;
    for (int x = 0; x < cur.n; ++x) {
      const int gl = cur.g[x] / 2, gr = cur.g[x] - gl;
      if (gl > 1) {
        nxt.s[nxt.n] = cur.s[x];
        nxt.g[nxt.n++] = gl;
      }
      if (gr > 1) {
        nxt.s[nxt.n] = cur.s[x] + gl;
        nxt.g[nxt.n++] = gr;
      }
    }
    cur = nxt;
  }
  hipLaunchKernelGGL(group_sort_kernel, dim3(N / C, bh), dim3(kThreads), 0, s, N, C, groups_out);
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
  // Key-tile slices per group: the group's queries are gathered once per
  // workgroup and reused over its slice of the keys.  About 6144 workgroups in
  // all (t2i, 3168 groups: two slices) balance that gather against filling the
  // chip; at most four slices.
  const int64_t n_groups = int64_t(B) * H * G;
  const int64_t slices = std::min<int64_t>(std::min(4, (N + 127) / 128),
                                           std::max<int64_t>(1, (6144 + n_groups / 2) / n_groups));
  const dim3 grid(static_cast<uint32_t>(n_groups), static_cast<uint32_t>(slices));
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
