// Block-sparse FlashAttention forward for gfx950 (MI355X).
//
// BSA-DiT §4.1: the FlashAttention tile loop keeps its outer loop over query
// blocks, and its inner loop visits only the KV blocks listed for that query
// block in a compact index read from global memory (here CSR).  BSA-DiT §4.3:
// the online softmax is carried over the visited blocks only and divided by
// their true total at the end, which is exactly the softmax with skipped
// blocks at -inf.
//
// Kernel design (one workgroup per CSR row = one query block of one head):
//   * 2*BLK/32 wavefronts: BLK/32 query groups of 32 rows times 2 key halves.
//     Wave (g, h) keeps its own online-softmax state for query rows
//     32g..32g+31 over keys h*BLK/2 .. (h+1)*BLK/2-1 of every visited tile;
//     the two halves are merged through LDS once, after the last tile.  This
//     halves both the serial chain of each wave and the registers it needs.
//   * Per active KV block: K [BLK x D] row-major and V^T [D x BLK] are staged
//     in LDS, double buffered, from 16-byte buffer loads issued one tile ahead
//     (register staging: half of the waves fetch K, the other half V), so one
//     barrier per tile.  Buffer bounds turn keys past N and invalid columns
//     into zeros without branches.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the accumulator of a lane holds
//     16 keys of ONE query, so row max / row sum are in-lane plus one
//     cross-half exchange, and P^T leaves the accumulator already in the
//     B-operand layout of the next product.
//   * O^T += V^T P^T on the same MFMA; V^T is stored with bits 2 and 3 of the
//     key index swapped inside each 16-key group, which puts the 8 keys a lane
//     needs for one MFMA step in 16 contiguous bytes.
//   * Softmax in the exp2 domain with scale*log2(e) folded into one FMA;
//     fp32 state (m, l, acc); the running sum stays lane-partial until the
//     epilogue; the accumulator is rescaled only when a row maximum grows by
//     more than 2^8 (exact: the final division uses the same stale maximum);
//     P is rounded to bf16 only as the MFMA operand.
//   * A partial last block masks keys >= N to -inf and stores no query row
//     >= N.  Columns outside [0, nb) contribute nothing.
#include <math.h>

#include <mutex>

#include "common.h"

namespace bsa {
namespace {

template <int BLK, int HD>
struct FwdCfg {
  static constexpr int NQG = BLK / 32;            // query groups of 32 rows
  static constexpr int NW = 2 * NQG;              // wavefronts: query group x key half
  static constexpr int NT = 64 * NW;              // threads per workgroup (= 4 * BLK)
  static constexpr int KS = HD + 8;               // LDS row stride of K (bf16 elements)
  static constexpr int VS = BLK + 8;              // LDS row stride of V^T (bf16 elements)
  static constexpr int K_ELEMS = BLK * KS;
  static constexpr int V_ELEMS = HD * VS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;  // bf16 elements per pipeline stage
  static constexpr size_t LDS_BYTES = size_t(2) * STAGE * 2;
  static constexpr int CPR = HD / 8;               // 16-byte chunks per token row
  static constexpr int KCH = BLK * CPR / (NT / 2); // K chunks per K-loading thread
  static constexpr int VQ = BLK * CPR / 4 / (NT / 2);  // V quads per V-loading thread
  static constexpr int NDC = HD / 16;              // k-steps of the QK^T product
  static constexpr int NKT = BLK / 64;             // 32-key subtiles per key half
  static constexpr int NDT = HD / 32;              // 32-wide d subtiles of the output
  static_assert(KCH * (NT / 2) == BLK * CPR, "K chunks must divide evenly");
  static_assert(VQ * (NT / 2) * 4 == BLK * CPR, "V quads must divide evenly");
  // Merge area (reuses the stage buffers): per query group 64 lanes x (acc + m + l).
  static constexpr size_t MERGE_BYTES = size_t(NQG) * 64 * (NDT * 16 + 4) * 4;
  static_assert(MERGE_BYTES <= LDS_BYTES, "merge area must fit in the stage buffers");
};

// Position of key kv inside a V^T row: bits 2 and 3 swapped.
__device__ __forceinline__ int kv_perm(int kv) {
  return (kv & ~12) | ((kv & 4) << 1) | ((kv & 8) >> 1);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const uint16_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
  const uint16_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(b));
  return uint32_t(lo) | (uint32_t(hi) << 16);
}

// Buffer resource over [base, base + bytes): loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Value of lane l ^ 32 (the other half of the wavefront), without LDS.
__device__ __forceinline__ float other_half(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  // Lanes < 32 receive the upper half in the second result, lanes >= 32 the
  // lower half in the first.
  return __uint_as_float((threadIdx.x & 32) ? sw[0] : sw[1]);
}

// Largest growth of the running max (log2 units) tolerated before the
// accumulator is rescaled; probabilities then stay below 2^8 before the final
// division, well inside fp32 and bf16 range.
constexpr float kRescaleSlack = 8.0f;

template <int BLK, int HD>
__global__ __launch_bounds__(4 * BLK) void fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, const int32_t* __restrict__ work, int32_t N,
    int32_t nb, int32_t n_rows, float sl2, uint16_t* __restrict__ O, float* __restrict__ LSE,
    float* __restrict__ part) {
  using C = FwdCfg<BLK, HD>;
  extern __shared__ __align__(16) uint16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qg = wave % C::NQG;  // query group
  const int kh = wave / C::NQG;  // key half
  const int ql = lane & 31;      // query column of this lane in the MFMA tiles
  const int hh = lane >> 5;      // which half of the k / row dimension the lane feeds

  // Work item: tiles [tb, te) of row r; slot >= 0 sends a partial result to
  // the workspace instead of O (the row was cut into chunks).
  int r, tb = 0, te = INT32_MAX, slot = -1;
  if (work) {
    const int4 it = *reinterpret_cast<const int4*>(work + 4 * size_t(blockIdx.x));
    r = it.x;
    tb = it.y;
    te = it.z;
    slot = it.w;
  } else {
    r = static_cast<int>(blockIdx.x);
  }
  if (r < 0 || r >= n_rows) return;
  const int bh = r / nb;
  const int qb = r - bh * nb;
  const size_t head = size_t(bh) * size_t(N) * HD;
  const uint32_t head_bytes = static_cast<uint32_t>(size_t(N) * HD * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + head, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + head, head_bytes);

  const int nnz = row_ptr[n_rows];
  int start = row_ptr[r];
  int end = row_ptr[r + 1];
  start = min(max(start, 0), nnz);
  end = min(max(end, start), nnz);
  tb = max(tb, 0);
  te = min(te, end - start);
  start += tb;
  const int cnt = max(te - tb, 0);

  // Query fragment (B operand of S^T = K Q^T): lane holds d = 16c + 8hh .. +7.
  // Rows past N read as zeros through the buffer bound.
  const int qrow = qb * BLK + qg * 32 + ql;
  bf16x8 qf[C::NDC];
  {
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + head, head_bytes);
    const uint32_t qoff = static_cast<uint32_t>(qrow) * HD * 2;
#pragma unroll
    for (int c = 0; c < C::NDC; ++c)
      qf[c] = __builtin_bit_cast(bf16x8, buf_load16(qrs, qoff + (2 * c + hh) * 16));
  }
  // Retire the query loads here: otherwise the wait-count bookkeeping still sees
  // them pending inside the tile loop and drains the K/V prefetch before every
  // product.  (vmcnt = 0, expcnt and lgkmcnt left at their maxima.)
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // Staging registers: threads [0, NT/2) fetch V quads, threads [NT/2, NT) fetch K.
  const bool loads_k = tid >= C::NT / 2;
  const int lt = loads_k ? tid - C::NT / 2 : tid;
  constexpr int NREG = C::KCH > 4 * C::VQ ? C::KCH : 4 * C::VQ;
  uint4 st[NREG];

  auto tile_valid = [&](int j) -> int {
    return (j >= 0 && j < nb) ? min(BLK, N - j * BLK) : 0;
  };

  // Global -> registers for KV block j.  Keys past N, and every key of a
  // column outside [0, nb), read as zeros through the buffer bound.
  auto load_tile = [&](int j) {
    const uint32_t tb = (j >= 0 && j < nb) ? static_cast<uint32_t>(j) * BLK * HD * 2 : head_bytes;
    if (loads_k) {
#pragma unroll
      for (int t = 0; t < C::KCH; ++t) {
        const int ch = lt + t * (C::NT / 2);
        const int row = ch / C::CPR;
        const int c8 = ch - row * C::CPR;
        st[t] = buf_load16(krs, tb + row * HD * 2 + c8 * 16);
      }
    } else {
#pragma unroll
      for (int t = 0; t < C::VQ; ++t) {
        const int qd = lt + t * (C::NT / 2);
        const int rq = qd % (BLK / 4);
        const int c8 = qd / (BLK / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          st[4 * t + e] = buf_load16(vrs, tb + (4 * rq + e) * HD * 2 + c8 * 16);
      }
    }
  };

  // Registers -> LDS: K row-major; V transposed, four keys per 8-byte store.
  auto store_tile = [&](int buf) {
    uint16_t* ks = smem + buf * C::STAGE;
    uint16_t* vt = ks + C::K_ELEMS;
    if (loads_k) {
#pragma unroll
      for (int t = 0; t < C::KCH; ++t) {
        const int ch = lt + t * (C::NT / 2);
        const int row = ch / C::CPR;
        const int c8 = ch - row * C::CPR;
        *reinterpret_cast<uint4*>(ks + row * C::KS + c8 * 8) = st[t];
      }
    } else {
#pragma unroll
      for (int t = 0; t < C::VQ; ++t) {
        // Consecutive lanes take consecutive key quads of one 8-column chunk, so
        // each 8-byte store of a half-wave lands on 64 distinct LDS banks.
        const int qd = lt + t * (C::NT / 2);
        const int rq = qd % (BLK / 4);
        const int c8 = qd / (BLK / 4);
        uint16_t* dst = vt + (c8 * 8) * C::VS + kv_perm(4 * rq);
        const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&st[4 * t + 0]);
        const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&st[4 * t + 1]);
        const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&st[4 * t + 2]);
        const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&st[4 * t + 3]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // d = 8*c8 + 2w takes the low halves, d + 1 the high halves.
          const uint2 even = make_uint2(__builtin_amdgcn_perm(r1[w], r0[w], 0x05040100u),
                                        __builtin_amdgcn_perm(r3[w], r2[w], 0x05040100u));
          const uint2 odd = make_uint2(__builtin_amdgcn_perm(r1[w], r0[w], 0x07060302u),
                                       __builtin_amdgcn_perm(r3[w], r2[w], 0x07060302u));
          *reinterpret_cast<uint2*>(dst + (2 * w) * C::VS) = even;
          *reinterpret_cast<uint2*>(dst + (2 * w + 1) * C::VS) = odd;
        }
      }
    }
  };

  float m_run = -INFINITY;  // running max of scale*log2(e)*s (possibly stale by < slack)
  float l_run = 0.f;        // lane-partial running sum
  f32x16 acc[C::NDT];
#pragma unroll
  for (int u = 0; u < C::NDT; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[u][i] = 0.f;

  // This wave's key half of one KV tile from LDS; keys >= valid (only in a
  // partial last block or an out-of-range column) are masked to -inf on a
  // rarely taken branch.
  auto compute_tile = [&](const uint16_t* ks, const uint16_t* vt, int valid) {
    const f32x16 zero = {};
    f32x16 s[C::NKT];
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) {
      const int key0 = (kh * C::NKT + kt) * 32;
#pragma unroll
      for (int c = 0; c < C::NDC; ++c) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(ks + (key0 + ql) * C::KS + 16 * c + 8 * hh);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], c == 0 ? zero : s[kt], 0, 0, 0);
      }
    }
    if (__builtin_expect(valid < BLK, 0)) {
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kv = (kh * C::NKT + kt) * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (kv >= valid) s[kt][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
    mx = fmaxf(mx, other_half(mx));
    const float mt = mx * sl2;
    // Lazy rescale: only when some row's max grew by more than the slack.
    const bool need = mt > m_run + kRescaleSlack;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;
      m_run = need ? mt : m_run;
      l_run *= alpha;
#pragma unroll
      for (int u = 0; u < C::NDT; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[u][i] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

    // Row sums in four independent chains (no long serial add dependency).
    float ls[4];
    bf16x8 pb[C::NKT][2];
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][i], sl2, -m_use));
        if (kt == 0 && i < 4)
          ls[i] = p;
        else
          ls[i & 3] += p;
        pb[kt][i >> 3][i & 7] = static_cast<__bf16>(p);
      }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);

    // O^T += V^T P^T: A = V^T rows d = 32u + ql, keys at permuted positions 8hh..8hh+7.
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int u = 0; u < C::NDT; ++u) {
          const int key0 = (kh * C::NKT + kt) * 32 + 16 * c2;
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(vt + (32 * u + ql) * C::VS + key0 + 8 * hh);
          acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kt][c2], acc[u], 0, 0, 0);
        }
  };

  // Tiles run in windows of 64: lane i of `colw` holds the window's column i
  // (one vector load per window, read back with v_readlane), so nothing the
  // inner loop carries from one tile to the next comes from memory.
  int t = 0;
  for (int w0 = 0; w0 < cnt; w0 += 64) {
    const int wn = min(64, cnt - w0);
    const int colw = lane < wn ? col_idx[start + w0 + lane] : -1;
    // First column of the next window, or this window's last if there is none.
    const int next_first = w0 + 64 < cnt ? col_idx[start + w0 + 64] : -1;
    // Retire the window load now (once per 64 tiles) so the inner loop never
    // has to drain the tile prefetch just to read a column index.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (w0 == 0) load_tile(__builtin_amdgcn_readfirstlane(colw));
    for (int u = 0; u < wn; ++u, ++t) {
      const int buf = t & 1;
      const int j = __builtin_amdgcn_readlane(colw, u);
      // Prefetch target: the next tile (the very last tile harmlessly reloads itself).
      const int jn = u + 1 < wn ? __builtin_amdgcn_readlane(colw, u + 1)
                                : (t + 1 < cnt ? next_first : j);
      store_tile(buf);
      __syncthreads();
      load_tile(jn);
      const uint16_t* ks = smem + buf * C::STAGE;
      compute_tile(ks, ks + C::K_ELEMS, tile_valid(j));
    }
  }

  // Merge the two key halves: wave (g, 1) hands (m, l, acc) to wave (g, 0).
  float l_half = l_run + other_half(l_run);
  __syncthreads();  // every wave is done reading the stage buffers
  float* mg = reinterpret_cast<float*>(smem) + size_t(qg) * 64 * (C::NDT * 16 + 4);
  if (kh == 1) {
#pragma unroll
    for (int u = 0; u < C::NDT; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(mg + ((u * 4 + g) * 64 + lane) * 4) =
            f32x4{acc[u][4 * g], acc[u][4 * g + 1], acc[u][4 * g + 2], acc[u][4 * g + 3]};
    mg[C::NDT * 16 * 64 + lane] = m_run;
    mg[C::NDT * 16 * 64 + 64 + lane] = l_half;
  }
  __syncthreads();
  if (kh == 1) return;
  {
    const float m1 = mg[C::NDT * 16 * 64 + lane];
    const float l1 = mg[C::NDT * 16 * 64 + 64 + lane];
    const float m = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
    l_half = l_half * a0 + l1 * a1;
    m_run = m;
#pragma unroll
    for (int u = 0; u < C::NDT; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(mg + ((u * 4 + g) * 64 + lane) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[u][4 * g + e] = acc[u][4 * g + e] * a0 + o1[e] * a1;
      }
  }

  if (slot >= 0) {
    // Partial result of one chunk: unnormalised acc, running max (log2 units)
    // and running sum, merged with the row's other chunks by merge_kernel.
    float* po = part + size_t(slot) * BLK * (HD + 2);
    const int q = qg * 32 + ql;
#pragma unroll
    for (int u = 0; u < C::NDT; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(po + q * HD + 32 * u + 8 * g + 4 * hh) =
            f32x4{acc[u][4 * g], acc[u][4 * g + 1], acc[u][4 * g + 2], acc[u][4 * g + 3]};
    if (hh == 0) {
      po[BLK * HD + q] = m_run;
      po[BLK * HD + BLK + q] = l_half;
    }
    return;
  }

  const float inv = l_half > 0.f ? 1.f / l_half : 0.f;
  if (qrow < N) {
    uint16_t* orow = O + head + size_t(qrow) * HD;
#pragma unroll
    for (int u = 0; u < C::NDT; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * u + 8 * g + 4 * hh;
        const uint32_t w0 = pack_bf16x2(acc[u][4 * g + 0] * inv, acc[u][4 * g + 1] * inv);
        const uint32_t w1 = pack_bf16x2(acc[u][4 * g + 2] * inv, acc[u][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d0) = make_uint2(w0, w1);
      }
    if (hh == 0 && LSE != nullptr) {
      LSE[size_t(bh) * N + qrow] =
          l_half > 0.f ? (m_run + __builtin_amdgcn_logf(l_half)) * 0.69314718055994531f
                       : -INFINITY;
    }
  }
}

// Combines the chunk partials of every cut row: with M = max_c m_c,
// O = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c and LSE = (M + log2 L) ln 2.
template <int BLK, int HD>
__global__ __launch_bounds__(256) void merge_kernel(const int32_t* __restrict__ merges,
                                                    const float* __restrict__ part, int32_t N,
                                                    int32_t nb, int32_t n_rows,
                                                    uint16_t* __restrict__ O,
                                                    float* __restrict__ LSE) {
  const int3 mg = *reinterpret_cast<const int3*>(merges + 3 * size_t(blockIdx.x));
  const int r = mg.x, slot0 = mg.y, nch = mg.z;
  if (r < 0 || r >= n_rows) return;
  const int bh = r / nb;
  const int qb = r - bh * nb;
  const size_t head = size_t(bh) * size_t(N) * HD;
  constexpr int D4 = HD / 4;
  for (int idx = threadIdx.x; idx < BLK * D4; idx += 256) {
    const int q = idx / D4;
    const int d = (idx - q * D4) * 4;
    const int qrow = qb * BLK + q;
    if (qrow >= N) continue;
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c)
      M = fmaxf(M, part[size_t(slot0 + c) * BLK * (HD + 2) + BLK * HD + q]);
    float L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
      for (int c = 0; c < nch; ++c) {
        const float* pc = part + size_t(slot0 + c) * BLK * (HD + 2);
        const float mc = pc[BLK * HD + q];
        const float w = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - M);
        L += w * pc[BLK * HD + BLK + q];
        const f32x4 oc = *reinterpret_cast<const f32x4*>(pc + q * HD + d);
        o += w * oc;
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    *reinterpret_cast<uint2*>(O + head + size_t(qrow) * HD + d) =
        make_uint2(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv));
    if (d == 0 && LSE != nullptr)
      LSE[size_t(bh) * N + qrow] =
          L > 0.f ? (M + __builtin_amdgcn_logf(L)) * 0.69314718055994531f : -INFINITY;
  }
}

template <int BLK, int HD>
bsa_status launch_fwd(const void* q, const void* k, const void* v, int32_t N, int32_t nb,
                      int32_t n_rows, const int32_t* row_ptr, const int32_t* col_idx,
                      const int32_t* work, int32_t n_items, int32_t n_merges, float sl2, void* o,
                      float* lse, float* part, hipStream_t stream) {
  using C = FwdCfg<BLK, HD>;
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_kernel<BLK, HD>),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(C::LDS_BYTES));
  });
  if (attr != hipSuccess) return BSA_ERR_HIP;
  const int32_t grid = work ? n_items : n_rows;
  if (grid > 0) {
    hipLaunchKernelGGL((fwd_kernel<BLK, HD>), dim3(grid), dim3(C::NT), C::LDS_BYTES, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), row_ptr, col_idx, work, N, nb, n_rows,
                       sl2, static_cast<uint16_t*>(o), lse, part);
    BSA_HIP_CHECK_LAUNCH();
  }
  if (work && n_merges > 0) {
    hipLaunchKernelGGL((merge_kernel<BLK, HD>), dim3(n_merges), dim3(256), 0, stream,
                       work + 4 * size_t(n_items), part, N, nb, n_rows,
                       static_cast<uint16_t*>(o), lse);
    BSA_HIP_CHECK_LAUNCH();
  }
  return BSA_OK;
}

}  // namespace
}  // namespace bsa

extern "C" BSA_API size_t bsa_forward_workspace_bytes(int32_t n_slots, int32_t D,
                                                      int32_t block) {
  if (n_slots < 0 || D < 1 || block < 1) return 0;
  return size_t(n_slots) * size_t(block) * size_t(D + 2) * sizeof(float);
}

extern "C" BSA_API bsa_status bsa_forward(const void* q, const void* k, const void* v,
                                          int32_t B, int32_t H, int32_t N, int32_t D,
                                          int32_t block, const int32_t* row_ptr_dev,
                                          const int32_t* col_idx_dev, const int32_t* work_dev,
                                          int32_t n_items, int32_t n_merges, int32_t n_slots,
                                          float scale, void* o, float* lse, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  using namespace bsa;
  if (!q || !k || !v || !o || !row_ptr_dev || !col_idx_dev) return BSA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return BSA_ERR_INVALID_ARG;
  if (!supported_shape(D, block)) return BSA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return BSA_ERR_INVALID_ARG;
  if (!(scale == scale)) return BSA_ERR_INVALID_ARG;
  const int32_t nb = n_blocks(N, block);
  // Buffer offsets inside one head are 32-bit: keep a head plus one tile below 2^31 bytes.
  if ((int64_t(nb) + 1) * block * D * 2 >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  const int64_t rows = int64_t(B) * H * nb;
  if (rows > INT32_MAX - 1) return BSA_ERR_UNSUPPORTED;
  const int32_t n_rows = static_cast<int32_t>(rows);
  if (work_dev) {
    if (!aligned16(work_dev) || n_items < 0 || n_merges < 0 || n_slots < 0)
      return BSA_ERR_INVALID_ARG;
    if (n_merges > 0) {
      if (!workspace || !aligned16(workspace)) return BSA_ERR_INVALID_ARG;
      if (workspace_bytes < bsa_forward_workspace_bytes(n_slots, D, block))
        return BSA_ERR_CAPACITY;
    }
  } else {
    n_items = n_merges = 0;
  }
  const float sc = scale > 0.f ? scale : 1.f / sqrtf(static_cast<float>(D));
  const float sl2 = sc * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(workspace);
#define BSA_FWD_ARGS                                                                            \
  q, k, v, N, nb, n_rows, row_ptr_dev, col_idx_dev, work_dev, n_items, n_merges, sl2, o, lse, \
      part, s
  if (block == 64 && D == 64) return launch_fwd<64, 64>(BSA_FWD_ARGS);
  if (block == 64 && D == 128) return launch_fwd<64, 128>(BSA_FWD_ARGS);
  if (block == 128 && D == 64) return launch_fwd<128, 64>(BSA_FWD_ARGS);
  return launch_fwd<128, 128>(BSA_FWD_ARGS);
#undef BSA_FWD_ARGS
}
