// Backward of block-sparse attention over the forward's CSR (BSA-DiT §2.3 and
// §5.2 train with the block mask; §4.1 and §4.3 define the forward: listed
// blocks visited, skipped blocks as -inf scores).  The gradient of
// O = softmax(scale Q K^T + M) V for an incoming dO, with the forward's LSE:
//   P = exp(scale q.k - LSE), dV = P^T dO, dP = dO V^T,
//   delta_t = sum_d dO[t,d] O[t,d], dS = P (dP - delta), dQ = scale dS K,
//   dK = scale dS^T Q.
// Four launches on the caller's stream:
//   prep       per query row (LSE * log2(e), delta), fp32;
//   transpose  per head, the query blocks that list each key block, ascending;
//   dkdv       one workgroup per key block, walking its query blocks;
//   dq         one workgroup per query block, walking its CSR row.
// The two gradient kernels recompute S and P from the LSE; neither uses atomics
// on the gradients, so results are deterministic.  Block 64 and D = 64.
#include <math.h>

#include <mutex>

#include "common.h"
#include "tile.h"

namespace bsa {
namespace {

constexpr int kBB = 64;     // block (query block = key block)
constexpr int kBD = 64;     // head dimension
constexpr int kRB = 128;    // bytes of one bf16 row
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void lds_write16(uint32_t addr, v4u x) {
  *reinterpret_cast<BSA_LDS v4u*>(static_cast<uintptr_t>(addr)) = x;
}

__device__ __forceinline__ v4u load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ float dot8(v4u a, v4u b) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = a[i], y = b[i];
    s = fmaf(__uint_as_float(x << 16), __uint_as_float(y << 16), s);
    s = fmaf(__uint_as_float(x & 0xffff0000u), __uint_as_float(y & 0xffff0000u), s);
  }
  return s;
}

// Per query row t: (LSE_t * log2(e), delta_t); rows with LSE = -inf (no active key)
// get +inf so that every probability of the row is exp2(-inf) = 0.  Eight lanes
// per row, 16 bytes each.
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ O,
                                                   const uint16_t* __restrict__ dO,
                                                   const float* __restrict__ LSE, int64_t rows,
                                                   float2* __restrict__ out) {
  const int64_t t = (int64_t(blockIdx.x) * 256 + threadIdx.x) >> 3;
  const int c = threadIdx.x & 7;
  float acc = 0.f;
  if (t < rows) {
    const v4u a = *reinterpret_cast<const v4u*>(O + t * kBD + 8 * c);
    const v4u b = *reinterpret_cast<const v4u*>(dO + t * kBD + 8 * c);
    acc = dot8(a, b);
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (c == 0 && t < rows) {
    const float l = LSE[t];
    out[t] = make_float2(l > -INFINITY ? l * kLog2e : INFINITY, acc);
  }
}

// Transpose of one head's CSR: for key block j, the query blocks i whose row
// lists j, ascending.  Head bh's entries keep the CSR's range
// [row_ptr[bh nb], row_ptr[(bh+1) nb]); column j starts at col_ptr[bh nb + j].
// A pair listed twice, or a column outside [0, nb), leaves a slot that is
// filled with -1 at the end of the head's last column.  An LDS bitmap
// (bit i of word j*W + i/32) orders each column without sorting.
__global__ __launch_bounds__(256) void transpose_kernel(const int32_t* __restrict__ row_ptr,
                                                        const int32_t* __restrict__ col_idx,
                                                        int32_t nb, int32_t n_heads,
                                                        int32_t* __restrict__ col_ptr,
                                                        int32_t* __restrict__ row_idx) {
  extern __shared__ uint32_t bits[];
  __shared__ int32_t start[kMaxBlocks];
  __shared__ int32_t tail_sh;
  const int tid = threadIdx.x;
  const int W = (nb + 31) >> 5;
  const int bh = blockIdx.x;
  const int r0 = bh * nb;
  for (int x = tid; x < nb * W; x += 256) bits[x] = 0u;
  __syncthreads();
  for (int i = tid; i < nb; i += 256) {
    const int e1 = row_ptr[r0 + i + 1];
    for (int e = row_ptr[r0 + i]; e < e1; ++e) {
      const int j = col_idx[e];
      if (j >= 0 && j < nb) atomicOr(&bits[j * W + (i >> 5)], 1u << (i & 31));
    }
  }
  __syncthreads();
  for (int j = tid; j < nb; j += 256) {
    int c = 0;
    for (int w = 0; w < W; ++w) c += __popc(bits[j * W + w]);
    start[j] = c;
  }
  __syncthreads();
  if (tid == 0) {
    int run = row_ptr[r0];
    for (int j = 0; j < nb; ++j) {
      const int c = start[j];
      start[j] = run;
      col_ptr[r0 + j] = run;
      run += c;
    }
    tail_sh = run;
    if (bh == n_heads - 1) col_ptr[r0 + nb] = row_ptr[r0 + nb];
  }
  __syncthreads();
  const int end = row_ptr[r0 + nb];
  for (int e = tail_sh + tid; e < end; e += 256) row_idx[e] = -1;
  for (int j = tid; j < nb; j += 256) {
    int pos = start[j];
    for (int w = 0; w < W; ++w) {
      uint32_t m = bits[j * W + w];
      while (m) {
        const int b = __builtin_ctz(m);
        m &= m - 1u;
        row_idx[pos++] = 32 * w + b;
      }
    }
  }
}

// dK, dV of one key block j (workgroup (bh, j), two wavefronts; wave w owns keys
// 32w .. 32w+31, which are the columns of its tiles).  For every query block i
// of the column: the 64 Q and dO rows are staged in LDS (swizzled), then per
// 32-query tile S = Q K^T and dP = dO V^T on MFMA (K, V rows of the wave's keys
// are the B operands, held in registers), P = exp2(S scale log2e - LSE log2e),
// dS = P (dP - delta), and dV^T += dO^T P, dK^T += Q^T dS with dO^T, Q^T read
// transposed from LDS.
__global__ __launch_bounds__(128) void dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float2* __restrict__ ld,
    const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ row_idx, int32_t N,
    int32_t nb, float c2, float scale, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV) {
  __shared__ __align__(16) uint8_t smem[2 * kBB * kRB + 2 * kBB * 4];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((BSA_LDS uint8_t*)smem));
  const uint32_t qs = lds0, dss = lds0 + kBB * kRB;
  float* lse_s = reinterpret_cast<float*>(smem + 2 * kBB * kRB);
  float* del_s = lse_s + kBB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hh = lane >> 5;
  const int r = blockIdx.x;
  const int bh = r / nb, j = r - bh * nb;
  const size_t head = size_t(bh) * size_t(N) * kBD;
  const uint32_t hbytes = static_cast<uint32_t>(N) * kRB;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q + head, hbytes);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(K + head, hbytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(V + head, hbytes);
  const __amdgpu_buffer_rsrc_t dr = make_rsrc(dO + head, hbytes);
  const int key = kBB * j + 32 * w + ql;
  const bool key_ok = key < N;
  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t off = uint32_t(key) * kRB + uint32_t(32 * c + 16 * hh);
    kf[c] = __builtin_bit_cast(bf16x8, load16(kr, off));
    vf[c] = __builtin_bit_cast(bf16x8, load16(vr, off));
  }
  f32x16 dk[2], dv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      dk[u][x] = 0.f;
      dv[u][x] = 0.f;
    }
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int e0 = __builtin_amdgcn_readfirstlane(col_ptr[r]);
  const int e1 = __builtin_amdgcn_readfirstlane(col_ptr[r + 1]);
  for (int e = e0; e < e1; ++e) {
    const int i = __builtin_amdgcn_readfirstlane(row_idx[e]);
    if (i < 0 || i >= nb) continue;
    __syncthreads();  // the previous block's LDS reads are done
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int idx = tid + 128 * x;
      const int rr = idx >> 3, cc = idx & 7;
      const uint32_t off = uint32_t(kBB * i + rr) * kRB + uint32_t(16 * cc);
      lds_write16(qs + swz<kRB>(rr, cc), load16(qr, off));
      lds_write16(dss + swz<kRB>(rr, cc), load16(dr, off));
    }
    if (tid < kBB) {
      const int t = kBB * i + tid;
      const float2 x = t < N ? ld[size_t(bh) * N + t] : make_float2(INFINITY, 0.f);
      lse_s[tid] = x.x;
      del_s[tid] = x.y;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const f32x16 zero = {};
      f32x16 s, dp;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 qa = lds_read16(qs + swz<kRB>(32 * g + ql, 2 * c + hh));
        const bf16x8 da = lds_read16(dss + swz<kRB>(32 * g + ql, 2 * c + hh));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[c], c == 0 ? zero : s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[c], c == 0 ? zero : dp, 0, 0, 0);
      }
      // register e of this lane: query 32g + 8(e/4) + 4hh + e%4, key `key`
      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 L = *reinterpret_cast<const f32x4*>(lse_s + 32 * g + 8 * m + 4 * hh);
        const f32x4 Dl = *reinterpret_cast<const f32x4*>(del_s + 32 * g + 8 * m + 4 * hh);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int ei = 4 * m + x;
          float p = __builtin_amdgcn_exp2f(fmaf(s[ei], c2, -L[x]));
          p = key_ok ? p : 0.f;
          pb[ei >> 3][ei & 7] = static_cast<__bf16>(p);
          sb[ei >> 3][ei & 7] = static_cast<__bf16>(p * (dp[ei] - Dl[x]));
        }
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int col = 32 * u + tr_col;
          const int r_lo = 32 * g + 16 * k2 + tr_row;
          const uint32_t clo = (col & 7) * 2;
          const v4s dlo = lds_read_tr(dss + swz<kRB>(r_lo, col >> 3) + clo);
          const v4s dhi = lds_read_tr(dss + swz<kRB>(r_lo + 8, col >> 3) + clo);
          const v4s qlo = lds_read_tr(qs + swz<kRB>(r_lo, col >> 3) + clo);
          const v4s qhi = lds_read_tr(qs + swz<kRB>(r_lo + 8, col >> 3) + clo);
          const bf16x8 ad = __builtin_bit_cast(bf16x8, __builtin_shufflevector(dlo, dhi, 0, 1, 2, 3, 4, 5, 6, 7));
          const bf16x8 aq = __builtin_bit_cast(bf16x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
          dv[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, pb[k2], dv[u], 0, 0, 0);
          dk[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, sb[k2], dk[u], 0, 0, 0);
        }
    }
  }
  // register e of dv[u], dk[u]: dimension 32u + 8(e/4) + 4hh + e%4 of key `key`
  if (key_ok) {
    uint16_t* vrow = dV + head + size_t(key) * kBD;
    uint16_t* krow = dK + head + size_t(key) * kBD;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * u + 8 * g4 + 4 * hh;
        *reinterpret_cast<uint2*>(vrow + d) =
            make_uint2(pack_bf16x2(dv[u][4 * g4], dv[u][4 * g4 + 1]),
                       pack_bf16x2(dv[u][4 * g4 + 2], dv[u][4 * g4 + 3]));
        *reinterpret_cast<uint2*>(krow + d) =
            make_uint2(pack_bf16x2(scale * dk[u][4 * g4], scale * dk[u][4 * g4 + 1]),
                       pack_bf16x2(scale * dk[u][4 * g4 + 2], scale * dk[u][4 * g4 + 3]));
      }
  }
}

// dQ of one query block i (workgroup (bh, i), two wavefronts; wave kh owns keys
// 32kh .. 32kh+31 of every key block of the row).  The forward's orientation:
// S^T = K Q^T and dP^T = V dO^T with the queries as columns (Q^T, dO^T B
// operands held in registers, one LSE and delta per lane), dS^T = P^T (dP^T -
// delta), and dQ^T += K^T dS^T with K^T read transposed from the wave's LDS
// area.  The two key halves are summed through LDS at the end.
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float2* __restrict__ ld,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int32_t N,
    int32_t nb, float c2, float scale, uint16_t* __restrict__ dQ) {
  __shared__ __align__(16) uint8_t smem[2 * 32 * kRB + 2 * 8192];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((BSA_LDS uint8_t*)smem));
  const int lane = threadIdx.x & 63;
  const int kh = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ql = lane & 31, hh = lane >> 5;
  const int r = blockIdx.x;
  const int bh = r / nb, i = r - bh * nb;
  const size_t head = size_t(bh) * size_t(N) * kBD;
  const uint32_t hbytes = static_cast<uint32_t>(N) * kRB;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q + head, hbytes);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(K + head, hbytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(V + head, hbytes);
  const __amdgpu_buffer_rsrc_t dr = make_rsrc(dO + head, hbytes);
  const uint32_t ks = lds0 + uint32_t(kh) * (32 * kRB);
  bf16x8 qf[2][4], df[2][4];
  float L[2], Dl[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int t = kBB * i + 32 * g + ql;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t off = uint32_t(t) * kRB + uint32_t(32 * c + 16 * hh);
      qf[g][c] = __builtin_bit_cast(bf16x8, load16(qr, off));
      df[g][c] = __builtin_bit_cast(bf16x8, load16(dr, off));
    }
    const float2 x = t < N ? ld[size_t(bh) * N + t] : make_float2(INFINITY, 0.f);
    L[g] = x.x;
    Dl[g] = x.y;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[g][u][x] = 0.f;
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int e0 = __builtin_amdgcn_readfirstlane(row_ptr[r]);
  const int e1 = __builtin_amdgcn_readfirstlane(row_ptr[r + 1]);
  for (int e = e0; e < e1; ++e) {
    const int j = __builtin_amdgcn_readfirstlane(col_idx[e]);
    if (j < 0 || j >= nb) continue;
    const int kbase = kBB * j + 32 * kh;  // first key of this wave's half
    // K rows of the wave's 32 keys into its LDS area (one wavefront's LDS
    // operations complete in order, so the previous block's reads are done).
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int rr = 8 * x + (lane >> 3);
      lds_write16(ks + swz<kRB>(rr, lane & 7),
                  load16(kr, uint32_t(kbase + rr) * kRB + uint32_t(16 * (lane & 7))));
    }
    bf16x8 va[4], ka[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      va[c] = __builtin_bit_cast(bf16x8, load16(vr, uint32_t(kbase + ql) * kRB + uint32_t(32 * c + 16 * hh)));
      ka[c] = lds_read16(ks + swz<kRB>(ql, 2 * c + hh));
    }
    bf16x8 sb[2][2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const f32x16 zero = {};
      f32x16 s, dp;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qf[g][c], c == 0 ? zero : s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[c], df[g][c], c == 0 ? zero : dp, 0, 0, 0);
      }
      // register x of this lane: key kbase + 8(x/4) + 4hh + x%4, query 32g + ql
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int kv = kbase + 8 * (x >> 2) + 4 * hh + (x & 3);
        float p = __builtin_amdgcn_exp2f(fmaf(s[x], c2, -L[g]));
        p = kv < N ? p : 0.f;
        sb[g][x >> 3][x & 7] = static_cast<__bf16>(p * (dp[x] - Dl[g]));
      }
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int col = 32 * u + tr_col;
        const uint32_t clo = (col & 7) * 2;
        const v4s lo = lds_read_tr(ks + swz<kRB>(16 * k2 + tr_row, col >> 3) + clo);
        const v4s hi = lds_read_tr(ks + swz<kRB>(16 * k2 + 8 + tr_row, col >> 3) + clo);
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int g = 0; g < 2; ++g)
          acc[g][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sb[g][k2], acc[g][u], 0, 0, 0);
      }
  }
  // Key-half sum: wave kh finishes query group kh and hands group 1 - kh over.
  float* xo = reinterpret_cast<float*>(smem + 2 * 32 * kRB);
  auto send = [&](const f32x16 (&a)[2]) {
    float* dst = xo + size_t(kh) * 2048;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<f32x4*>(dst + ((u * 4 + g4) * 64 + lane) * 4) =
            f32x4{a[u][4 * g4], a[u][4 * g4 + 1], a[u][4 * g4 + 2], a[u][4 * g4 + 3]};
  };
  auto finish = [&](const f32x16 (&a)[2]) {
    const int t = kBB * i + 32 * kh + ql;
    if (t >= N) return;
    const float* src = xo + size_t(1 - kh) * 2048;
    uint16_t* qrow = dQ + head + size_t(t) * kBD;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(src + ((u * 4 + g4) * 64 + lane) * 4);
        const int d = 32 * u + 8 * g4 + 4 * hh;
        *reinterpret_cast<uint2*>(qrow + d) =
            make_uint2(pack_bf16x2(scale * (a[u][4 * g4] + o1[0]), scale * (a[u][4 * g4 + 1] + o1[1])),
                       pack_bf16x2(scale * (a[u][4 * g4 + 2] + o1[2]), scale * (a[u][4 * g4 + 3] + o1[3])));
      }
  };
  if (kh == 0)
    send(acc[1]);
  else
    send(acc[0]);
  __syncthreads();
  if (kh == 0)
    finish(acc[0]);
  else
    finish(acc[1]);
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace
}  // namespace bsa

extern "C" BSA_API size_t bsa_backward_workspace_bytes(int32_t B, int32_t H, int32_t N,
                                                      int32_t block, int64_t nnz) {
  using namespace bsa;
  if (B < 1 || H < 1 || N < 1 || block < 1 || nnz < 0) return 0;
  const size_t rows = size_t(B) * H * N;
  const size_t nrow = size_t(B) * H * n_blocks(N, block);
  return round256(rows * sizeof(float2)) + round256((nrow + 1) * sizeof(int32_t)) +
         round256(size_t(nnz) * sizeof(int32_t));
}

extern "C" BSA_API bsa_status bsa_backward(const void* q, const void* k, const void* v,
                                           const void* o, const void* d_o, const float* lse,
                                           int32_t B, int32_t H, int32_t N, int32_t D,
                                           int32_t block, const int32_t* row_ptr,
                                           const int32_t* col_idx, int64_t nnz, float scale,
                                           void* dq, void* dk, void* dv, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  using namespace bsa;
  if (!q || !k || !v || !o || !d_o || !lse || !row_ptr || (!col_idx && nnz > 0) || !dq || !dk ||
      !dv || !workspace)
    return BSA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || nnz < 0 || !(scale == scale)) return BSA_ERR_INVALID_ARG;
  if (D != kBD || block != kBB) return BSA_ERR_UNSUPPORTED;
  const int32_t nb = n_blocks(N, block);
  if (nb > kMaxBlocks || int64_t(N) * kRB >= (int64_t(1) << 31) || nnz > INT32_MAX ||
      int64_t(B) * H * nb > INT32_MAX)
    return BSA_ERR_UNSUPPORTED;
  for (const void* p : {q, k, v, o, d_o, static_cast<const void*>(dq), static_cast<const void*>(dk),
                        static_cast<const void*>(dv), static_cast<const void*>(workspace)})
    if (!aligned16(p)) return BSA_ERR_INVALID_ARG;
  if (workspace_bytes < bsa_backward_workspace_bytes(B, H, N, block, nnz)) return BSA_ERR_CAPACITY;
  const int64_t rows = int64_t(B) * H * N;
  const int32_t n_heads = B * H;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float2* ld = reinterpret_cast<float2*>(ws);
  int32_t* col_ptr = reinterpret_cast<int32_t*>(ws + round256(size_t(rows) * sizeof(float2)));
  int32_t* row_idx = reinterpret_cast<int32_t*>(
      reinterpret_cast<uint8_t*>(col_ptr) + round256((size_t(n_heads) * nb + 1) * sizeof(int32_t)));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const float sc = scale > 0.f ? scale : 1.f / sqrtf(static_cast<float>(D));

  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&transpose_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               kMaxBlocks * (kMaxBlocks / 32) * 4);
  });
  if (attr != hipSuccess) return BSA_ERR_HIP;

  hipLaunchKernelGGL(prep_kernel, dim3(static_cast<uint32_t>((rows * 8 + 255) / 256)), dim3(256),
                     0, s, static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(d_o), lse,
                     rows, ld);
  BSA_HIP_CHECK_LAUNCH();
  const size_t bits_bytes = size_t(nb) * ((nb + 31) / 32) * 4;
  hipLaunchKernelGGL(transpose_kernel, dim3(n_heads), dim3(256), bits_bytes, s, row_ptr, col_idx,
                     nb, n_heads, col_ptr, row_idx);
  BSA_HIP_CHECK_LAUNCH();
  const float c2 = sc * kLog2e;
  hipLaunchKernelGGL(dkdv_kernel, dim3(n_heads * nb), dim3(128), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(d_o), ld,
                     col_ptr, row_idx, N, nb, c2, sc, static_cast<uint16_t*>(dk),
                     static_cast<uint16_t*>(dv));
  BSA_HIP_CHECK_LAUNCH();
  hipLaunchKernelGGL(dq_kernel, dim3(n_heads * nb), dim3(128), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(d_o), ld,
                     row_ptr, col_idx, N, nb, c2, sc, static_cast<uint16_t*>(dq));
  BSA_HIP_CHECK_LAUNCH();
  return BSA_OK;
}
