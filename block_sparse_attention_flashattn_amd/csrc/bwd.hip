// Backward of block-sparse attention over the forward's CSR (BSA-DiT §2.3 and
// §5.2 train with the block mask; §4.1 and §4.3 define the forward: listed
// blocks visited, skipped blocks as -inf scores).  The gradient of
// O = softmax(scale Q K^T + M) V for an incoming dO, with the forward's LSE:
//   P = exp(scale q.k - LSE), dV = P^T dO, dP = dO V^T,
//   delta_t = sum_d dO[t,d] O[t,d], dS = P (dP - delta), dQ = scale dS K,
//   dK = scale dS^T Q.
// Five launches on the caller's stream (six at head dim 128):
//   prep       per query row (LSE * log2(e), delta), fp32;
//   transpose  per head, the query blocks that list each key block, ascending,
//              the split of long key columns and query rows into chunks, and
//              the head's work items appended to its die's work lists;
//   tpos       (head dim 128) per CSR entry, its block pair's dS tile slot;
//   dkdv       persistent workgroups, one chunk of a key block's query blocks
//              per item;
//   dq         persistent workgroups, one chunk of a query block's CSR row per
//              item (at head dim 128 from the dS tiles dkdv stored);
//   reduce     per split block, the chunks' fp32 partials summed in chunk order.
// A column or row longer than the chunk length (twice the mean row length, at
// least 16) is cut into near-equal chunks so that a few long ones (text blocks,
// anchor columns) do not set the length of the launch.  The dK/dV kernel
// recomputes S and P from the LSE; at head dim 64 so does the dQ kernel, at
// head dim 128 it reads the dS tiles the dK/dV kernel stored.  Nothing uses
// atomics on the gradients, so results are deterministic.  D = 64 or 128 over
// 64-row blocks (a 128-row block CSR is refined to the 64-row CSR first).
#include <math.h>

#include <algorithm>

#include <mutex>
#include <type_traits>

#include "common.h"
#include "tile.h"
#include "dma.h"

namespace bsa {
namespace {

constexpr int kBB = 64;     // block (query block = key block)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kDqStages = 2;  // K/V ring depth of the dQ kernel

// Work lists of the gradient kernels: one per die (XCD) when there are at least
// as many heads as dies, else one.  Head bh's items go to list bh % n_lists.
constexpr int kLists = 8;
constexpr int kClaimStride = 32;  // ints between two claim counters (own cache lines)
// Counter area (ints): [0], [1] partial-slot counters (dK/dV, dQ); kLenKv + l and
// kLenKv + kLists + l the chunk and whole-block items in dK/dV list l, kLenQ + l
// and kLenQ + kLists + l those of dQ list l; the claim counters of list l at
// kClaimKv + l kClaimStride and kClaimQ + l kClaimStride.  prep_kernel clears it.
constexpr int kLenKv = 16, kLenQ = 32, kClaimKv = 64, kClaimQ = kClaimKv + kLists * kClaimStride;
constexpr int kCtrInts = kClaimQ + kLists * kClaimStride;

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
// get +inf so that every probability of the row is exp2(-inf) = 0.  HD / 8 lanes
// per row, 16 bytes each.  Also clears the counter area of the later launches.
template <int HD>
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ O,
                                                   const uint16_t* __restrict__ dO,
                                                   const float* __restrict__ LSE, int64_t rows,
                                                   float2* __restrict__ out,
                                                   int32_t* __restrict__ slot_ctr) {
  if (blockIdx.x == 0)
    for (int x = threadIdx.x; x < kCtrInts; x += 256) slot_ctr[x] = 0;
  constexpr int LPR = HD / 8;  // lanes per row
  const int64_t t = (int64_t(blockIdx.x) * 256 + threadIdx.x) / LPR;
  const int c = threadIdx.x & (LPR - 1);
  float acc = 0.f;
  if (t < rows) {
    const v4u a = *reinterpret_cast<const v4u*>(O + t * HD + 8 * c);
    const v4u b = *reinterpret_cast<const v4u*>(dO + t * HD + 8 * c);
    acc = dot8(a, b);
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m);
  if (c == 0 && t < rows) {
    const float l = LSE[t];
    out[t] = make_float2(l > -INFINITY ? l * kLog2e : INFINITY, acc);
  }
}

// 4 bytes per lane from buffer offset `voff` into LDS at lds + 4 * lane (each
// dword checked against the buffer's range on its own).
__device__ __forceinline__ void dma4(v4i desc, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(desc)
      : "memory");
}

// Buffer descriptor with wave-uniform (scalar) fields.
__device__ __forceinline__ v4i uniform_desc(const void* base, uint32_t bytes) {
  v4i d = make_desc(base, bytes);
#pragma unroll
  for (int w = 0; w < 4; ++w) d[w] = __builtin_amdgcn_readfirstlane(d[w]);
  return d;
}

// A 32-row half tile (rows h0 .. h0 + 31 of a 64-row tile of RB-byte rows) is
// HALF_SEGS 1-KiB segments; lane l of segment s moves the 16-byte chunk that
// lands at its swizzled LDS position: row h0 + s * 1024 / RB + l / (RB / 16),
// position l % (RB / 16).  off[s] is its source offset from the half's first
// row, less 1024 (s % 4) (>= 0: segment s starts s KiB into the half), as
// dma16x4 takes it.
template <int RB>
__device__ __forceinline__ void half_offsets(int lane, int h0, uint32_t (&off)[RB / 32]) {
  constexpr int CPR = RB / 16, RPS = 1024 / RB;
#pragma unroll
  for (int s = 0; s < RB / 32; ++s) {
    const int r = s * RPS + lane / CPR, p = lane % CPR;
    off[s] = uint32_t(r) * RB + uint32_t((p ^ chunk_swizzle<RB>(h0 + r)) << 4) -
             uint32_t(s & 3) * 1024u;
  }
}
// The half tile at source offset tb of `desc` into LDS at dst (its segments
// consecutive), from half_offsets.
template <int RB>
__device__ __forceinline__ void dma_half_tile(v4i desc, const uint32_t (&off)[RB / 32],
                                              uint32_t tb, uint32_t dst) {
#pragma unroll
  for (int s = 0; s < RB / 32; s += 4)
    dma16x4(desc, tb + off[s], tb + off[s + 1], tb + off[s + 2], tb + off[s + 3],
            dst + uint32_t(s) * 1024u);
}

// The entries idx[e] of a CSR range [e0, e1) a workgroup walks in order, 64 at a
// time in one VGPR (lane l holds idx[base + l]); -1 past e1.
struct IndexWindow {
  const int32_t* idx;
  int e1, base, v;
  __device__ void init(const int32_t* p, int e0, int end, int lane) {
    idx = p;
    e1 = end;
    base = e0;
    v = e0 + lane < e1 ? idx[e0 + lane] : -1;
    asm volatile("" ::"v"(v));  // complete here, not inside a DMA-pipelined loop
  }
  // Entry e (e >= base, called with non-decreasing e).
  __device__ int at(int e, int lane) {
    if (e >= e1) return -1;
    if (e - base >= 64) {
      base += 64;
      v = base + lane < e1 ? idx[base + lane] : -1;
      asm volatile("" ::"v"(v));
    }
    return __builtin_amdgcn_readlane(v, e - base);
  }
};

// Number of chunks of a column or row of `len` entries: 1 up to the chunk
// length, else ceil(len / chunk) capped at max_ch.
__device__ __forceinline__ int n_chunks(int len, int chunk, int max_ch) {
  return len > chunk ? min((len + chunk - 1) / chunk, max_ch) : 1;
}

// Exclusive prefix sums of a[0, n) and, when b is not null, of b[0, n), in place,
// by a 256-thread workgroup (n <= 1024); returns the totals.  Each thread takes
// a run of consecutive entries, each wavefront scans its threads' sums with
// lane shifts, and one barrier shares the four wavefront totals.  Entries must
// be written before a barrier that precedes the call; the call ends with one.
// tmp: 8 ints of LDS.
__device__ int2 block_scan(int32_t* a, int32_t* b, int n, int32_t* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (n + 255) >> 8;
  const int lo = min(tid * per, n), hi = min(lo + per, n);
  int sa = 0, sb = 0;
  for (int x = lo; x < hi; ++x) {
    sa += a[x];
    if (b) sb += b[x];
  }
  int ia = sa, ib = sb;  // inclusive scans over the wavefront's threads
  for (int d = 1; d < 64; d <<= 1) {
    const int ta = __shfl_up(ia, d, 64), tb = __shfl_up(ib, d, 64);
    if (lane >= d) {
      ia += ta;
      ib += tb;
    }
  }
  if (lane == 63) {
    tmp[w] = ia;
    tmp[4 + w] = ib;
  }
  __syncthreads();
  int oa = ia - sa, ob = ib - sb, ta = 0, tb = 0;
  for (int v = 0; v < 4; ++v) {
    const int xa = tmp[v], xb = tmp[4 + v];
    if (v < w) {
      oa += xa;
      ob += xb;
    }
    ta += xa;
    tb += xb;
  }
  for (int x = lo; x < hi; ++x) {
    const int va = a[x];
    a[x] = oa;
    oa += va;
    if (b) {
      const int vb = b[x];
      b[x] = ob;
      ob += vb;
    }
  }
  __syncthreads();
  return make_int2(ta, tb);
}

// Transpose of one head's CSR: for key block j, the query blocks i whose row
// lists j, ascending.  Head bh's entries keep the CSR's range
// [row_ptr[bh nb], row_ptr[(bh+1) nb]); column j starts at col_ptr[bh nb + j].
// A pair listed twice, or a column outside [0, nb), leaves a slot that is
// filled with -1 at the end of the head's last column.  An LDS bitmap
// (bit i of word j*W + i/32) orders each column without sorting; the entries
// are read in parallel, in one run of consecutive entries per thread.
// Splits: col_split[bh nb + j] = (first partial slot, chunks) of key column j,
// row_split the same for the CSR rows; a head's split blocks take consecutive
// slots from the counters (cleared by prep_kernel).  If the slots run out (they
// cannot when the capacity is the bound the host sizes), the head is left
// unsplit, which is slower but exact.
// Work items: a record {bh nb + j, first entry, end entry, partial slot or -1}
// for every chunk of key column j (dK/dV list, entries of row_idx) and of CSR
// row j (dQ list, entries of col_idx), appended to list bh % n_lists at ranges
// the head reserves there.  A list has two parts of list_cap records: the
// chunks of split blocks (the longest items, claimed first), each head's in
// block order, and the whole blocks, each head's longest first (a counting
// sort by length; equal lengths in any order).
__global__ __launch_bounds__(256) void transpose_kernel(const int32_t* __restrict__ row_ptr,
                                                        const int32_t* __restrict__ col_idx,
                                                        int32_t nb, int32_t n_heads,
                                                        int32_t* __restrict__ col_ptr,
                                                        int32_t* __restrict__ row_idx,
                                                        int32_t chunk, int32_t max_ch,
                                                        int32_t* __restrict__ slot_ctr,
                                                        int32_t cap_kv, int32_t cap_q,
                                                        int2* __restrict__ col_split,
                                                        int2* __restrict__ row_split,
                                                        int32_t n_lists, int32_t list_cap,
                                                        int4* __restrict__ items_kv,
                                                        int4* __restrict__ items_q) {
  extern __shared__ uint32_t bits[];
  __shared__ int32_t rp[kMaxBlocks + 1];
  __shared__ int32_t start[kMaxBlocks], nch_c[kMaxBlocks], nch_r[kMaxBlocks];
  __shared__ int32_t pre_c[kMaxBlocks], pre_r[kMaxBlocks], tmp[8];
  __shared__ int32_t hist[kMaxBlocks];  // length histogram of the whole blocks
  __shared__ int32_t base_sh[4];
  const int tid = threadIdx.x;
  const int W = (nb + 31) >> 5;
  const int bh = blockIdx.x;
  const int r0 = bh * nb;
  for (int x = tid; x < nb * W; x += 256) bits[x] = 0u;
  for (int i = tid; i <= nb; i += 256) rp[i] = row_ptr[r0 + i];
  __syncthreads();
  const int begin = rp[0], end = rp[nb];
  for (int i = tid; i < nb; i += 256) {
    const int n = n_chunks(rp[i + 1] - rp[i], chunk, max_ch);
    nch_r[i] = n;
    pre_r[i] = n > 1 ? n : 0;
  }
  {
    // Thread tid sets the bits of a run of consecutive entries: one binary
    // search for the row of its first entry, then the row advances with the
    // entries; column indices are loaded eight at a time.
    const int per = (end - begin + 255) >> 8;
    int e = begin + tid * per;
    const int e_end = min(e + per, end);
    int row = 0;
    if (e < e_end) {
      int lo = 0, hi = nb - 1;  // the row i with rp[i] <= e < rp[i + 1]
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (rp[mid] <= e)
          lo = mid;
        else
          hi = mid - 1;
      }
      row = lo;
    }
    for (; e < e_end; e += 8) {
      int jv[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) jv[t] = e + t < e_end ? col_idx[e + t] : -1;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (e + t >= e_end) break;
        while (rp[row + 1] <= e + t) ++row;
        const int j = jv[t];
        if (j >= 0 && j < nb) atomicOr(&bits[j * W + (row >> 5)], 1u << (row & 31));
      }
    }
  }
  __syncthreads();
  for (int j = tid; j < nb; j += 256) {
    int c = 0;
    for (int w = 0; w < W; ++w) c += __popc(bits[j * W + w]);
    start[j] = c;
    nch_c[j] = c;  // the column's length (the last one gains the padding below)
  }
  __syncthreads();
  const int listed = block_scan(start, nullptr, nb, tmp).x;
  if (tid == 0) nch_c[nb - 1] += (end - begin) - listed;  // the head's -1 padding
  __syncthreads();
  for (int j = tid; j < nb; j += 256) {
    const int n = n_chunks(nch_c[j], chunk, max_ch);
    nch_c[j] = n;
    pre_c[j] = n > 1 ? n : 0;
  }
  __syncthreads();
  const int2 tot = block_scan(pre_c, pre_r, nb, tmp);
  const int tot_kv = tot.x, tot_q = tot.y;
  if (tid == 0) {
    int bk = tot_kv ? atomicAdd(slot_ctr, tot_kv) : 0;
    int bq = tot_q ? atomicAdd(slot_ctr + 1, tot_q) : 0;
    base_sh[0] = (bk < 0 || bk > cap_kv - tot_kv) ? -1 : bk;
    base_sh[1] = (bq < 0 || bq > cap_q - tot_q) ? -1 : bq;
    if (bh == n_heads - 1) col_ptr[r0 + nb] = end;
  }
  __syncthreads();
  const int bk = base_sh[0], bq = base_sh[1];
  for (int j = tid; j < nb; j += 256) {
    col_ptr[r0 + j] = begin + start[j];
    col_split[r0 + j] = (nch_c[j] > 1 && bk >= 0) ? make_int2(bk + pre_c[j], nch_c[j])
                                                  : make_int2(-1, 1);
    row_split[r0 + j] = (nch_r[j] > 1 && bq >= 0) ? make_int2(bq + pre_r[j], nch_r[j])
                                                  : make_int2(-1, 1);
  }
  __syncthreads();
  for (int j = tid; j < nb; j += 256) {  // 1 for the blocks left whole
    nch_c[j] = (nch_c[j] > 1 && bk >= 0) ? 0 : 1;
    nch_r[j] = (nch_r[j] > 1 && bq >= 0) ? 0 : 1;
  }
  __syncthreads();
  const int2 n_w = block_scan(nch_c, nch_r, nb, tmp);  // whole blocks before block j
  const int n_wk = n_w.x, n_wq = n_w.y;
  const int l = bh % n_lists;
  if (tid == 0) {
    // chunks: one per partial slot, at the slot's offset in the head's range
    base_sh[0] = atomicAdd(slot_ctr + kLenKv + l, bk >= 0 ? tot_kv : 0);
    base_sh[1] = atomicAdd(slot_ctr + kLenKv + kLists + l, n_wk);
    base_sh[2] = atomicAdd(slot_ctr + kLenQ + l, bq >= 0 ? tot_q : 0);
    base_sh[3] = atomicAdd(slot_ctr + kLenQ + kLists + l, n_wq);
  }
  __syncthreads();
  int4* const ck = items_kv + size_t(2 * l) * list_cap + base_sh[0];
  int4* const wk = items_kv + size_t(2 * l + 1) * list_cap + base_sh[1];
  int4* const cq = items_q + size_t(2 * l) * list_cap + base_sh[2];
  int4* const wq = items_q + size_t(2 * l + 1) * list_cap + base_sh[3];
  // Bin of a whole block of `len` entries: longer blocks in lower bins.
  auto bin = [](int len) { return kMaxBlocks - 1 - min(len, kMaxBlocks - 1); };
  for (int kind = 0; kind < 2; ++kind) {  // key columns, then CSR rows
    const int32_t* whole = kind ? nch_r : nch_c;
    const int n_whole = kind ? n_wq : n_wk;
    for (int b = tid; b < kMaxBlocks; b += 256) hist[b] = 0;
    __syncthreads();
    for (int j = tid; j < nb; j += 256) {
      const int len = kind ? rp[j + 1] - rp[j]
                           : (j + 1 < nb ? begin + start[j + 1] : end) - (begin + start[j]);
      if ((j + 1 < nb ? whole[j + 1] : n_whole) > whole[j]) atomicAdd(&hist[bin(len)], 1);
    }
    __syncthreads();
    block_scan(hist, nullptr, kMaxBlocks, tmp);
    for (int j = tid; j < nb; j += 256) {
      const int a = kind ? rp[j] : begin + start[j];
      const int len = (kind ? rp[j + 1] : (j + 1 < nb ? begin + start[j + 1] : end)) - a;
      if ((j + 1 < nb ? whole[j + 1] : n_whole) > whole[j]) {
        (kind ? wq : wk)[atomicAdd(&hist[bin(len)], 1)] = make_int4(r0 + j, a, a + len, -1);
      } else {
        const int n = n_chunks(len, chunk, max_ch), pre = kind ? pre_r[j] : pre_c[j];
        const int base = kind ? bq : bk;
        for (int c = 0; c < n; ++c)
          (kind ? cq : ck)[pre + c] = make_int4(r0 + j, a + int(int64_t(len) * c / n),
                                                a + int(int64_t(len) * (c + 1) / n), base + pre + c);
      }
    }
    __syncthreads();
  }
  for (int e = begin + listed + tid; e < end; e += 256) row_idx[e] = -1;
  for (int j = tid; j < nb; j += 256) {
    int pos = begin + start[j];
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

// Transposed position of every CSR entry of row r (its pair's slot in row_idx:
// the column's first slot plus the rows before r that list the column; -1 for
// a column outside [0, nb)), for dq_stored_kernel.  One wavefront per CSR row,
// a lane per entry, each a binary search over its column's ascending rows (the
// head's padding slots, -1, sit after the last column's rows and compare as
// larger than every row).
__global__ __launch_bounds__(64) void tpos_kernel(const int32_t* __restrict__ row_ptr,
                                                  const int32_t* __restrict__ col_idx,
                                                  const int32_t* __restrict__ col_ptr,
                                                  const int32_t* __restrict__ row_idx, int32_t nb,
                                                  int32_t* __restrict__ tpos) {
  const int r = blockIdx.x;
  const int bh = r / nb, i = r - bh * nb;
  const int b0 = row_ptr[r], b1 = row_ptr[r + 1];
  for (int e = b0 + static_cast<int>(threadIdx.x); e < b1; e += 64) {
    const int j = col_idx[e];
    int t = -1;
    if (j >= 0 && j < nb) {
      int lo = col_ptr[bh * nb + j], hi = col_ptr[bh * nb + j + 1];  // first slot holding >= i
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const int v = row_idx[mid];
        if (v >= 0 && v < i)
          lo = mid + 1;
        else
          hi = mid;
      }
      t = lo;
    }
    tpos[e] = t;
  }
}

// Persistent gradient workgroups take their items from the work lists:
// workgroup b starts at list b % n_lists (its own die's when there is one list
// per die: workgroups are dealt to the dies round robin); once that list is
// used up it reads every list's claim counter in one go and moves on to the
// next list with items left, so dies that finish early help the others.  One
// lane claims (vector atomics, agent scope); the claim for the next item is
// issued when an item starts, and its record is loaded during the item's last
// step.
struct ListClaims {
  const int4* items;
  const int32_t* lens;
  int32_t* claims;
  int n_lists, cap, list, nc, nw;  // nc, nw: the current list's chunks and whole blocks

  __device__ void load_lens() {
    nc = lens[list];
    nw = lens[kLists + list];
  }
  __device__ int claim() const {
    return __hip_atomic_fetch_add(claims + list * kClaimStride, 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  }
  // Called by all lanes of one wave: the item of claim number s (lane 0's) on
  // the current list (its chunks, then its whole blocks), else one claimed from a
  // list with items left; a record with block -1 once no list has any.
  __device__ int4 item(int s, int lane) {
    s = __builtin_amdgcn_readfirstlane(s);
    for (;;) {
      if (s < nc) return items[size_t(2 * list) * cap + s];
      if (s < nc + nw) return items[size_t(2 * list + 1) * cap + (s - nc)];
      int left = 0;
      if (lane < n_lists)
        left = lens[lane] + lens[kLists + lane] -
               __hip_atomic_load(claims + lane * kClaimStride, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t m = __ballot(left > 0);
      if (m == 0) return make_int4(-1, 0, 0, -1);
      const uint64_t hi = m >> list;  // lists at or after the current one first
      list = hi ? list + __builtin_ctzll(hi) : __builtin_ctzll(m);
      load_lens();
      int t = 0;
      if (lane == 0) t = claim();
      s = __builtin_amdgcn_readfirstlane(t);
    }
  }
};

// dK, dV of one chunk of key block j (item (bh, j, chunk), two wavefronts;
// wave w owns keys 32w .. 32w+31, which are the columns of its tiles).  For
// every query block i of the chunk: the 64 Q and dO rows are staged in LDS (swizzled), then per
// 32-query tile S = Q K^T and dP = dO V^T on MFMA (K, V rows of the wave's keys
// are the B operands, held in registers), P = exp2(S scale log2e - LSE log2e),
// dS = P (dP - delta), and dV^T += dO^T P, dK^T += Q^T dS with dO^T, Q^T read
// transposed from LDS.  With STORE, dS is also stored, bf16, as the pair's
// 64 x 64 tile (slot = its position in row_idx), for dq_stored_kernel.  An unsplit column
// writes bf16 dK, dV; a chunk of a split one writes its fp32 sums (dK
// unscaled) to the item's partial slot.
// At HD = 128 the two stages take 65 KiB of LDS: two workgroups per CU, one
// wave per SIMD, which may then use the whole register file.
template <int HD>
struct DkdvCfg {
  static constexpr int RB = HD * 2, NDC = HD / 16, NDT = HD / 32;
  static constexpr uint32_t kTile = kBB * RB, kHalf = kTile / 2, kLd = kBB * 8;
  static constexpr uint32_t kStage = 2 * kTile + kLd;
  static constexpr size_t kClaimAt = 2 * size_t(kStage);  // two records: the claimed items
  static constexpr size_t LDS_BYTES = kClaimAt + 32;
};

template <int HD, bool STORE>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(HD == 64 ? 2 : 1))) void dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float2* __restrict__ ld,
    const int32_t* __restrict__ row_idx,
    const int4* __restrict__ items, int32_t* __restrict__ ctr, int32_t n_lists, int32_t list_cap,
    int32_t N, int32_t nb, float c2, float scale, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, float* __restrict__ part, uint16_t* __restrict__ dst_tiles) {
  // Two stages of (Q tile, dO tile, per-row (LSE log2 e, delta)) of one query
  // block, each wave streaming its 32-row halves by LDS DMA one block ahead.
  using C = DkdvCfg<HD>;
  constexpr int RB = C::RB, NDC = C::NDC, NDT = C::NDT;
  constexpr uint32_t kTile = C::kTile, kHalf = C::kHalf, kLd = C::kLd, kStage = C::kStage;
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((BSA_LDS uint8_t*)smem));
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hh = lane >> 5;
  uint32_t hoff[RB / 32];
  half_offsets<RB>(lane, 32 * w, hoff);
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  ListClaims lc{items, ctr + kLenKv, ctr + kClaimKv, n_lists, list_cap,
                static_cast<int>(blockIdx.x % n_lists), 0, 0};
  int4* const claimed = reinterpret_cast<int4*>(smem + C::kClaimAt);
  int ticket = 0;
  int4 nxt = make_int4(-1, 0, 0, -1);  // wave 0: the next item, loaded in the last step
  if (tid < 64) {
    lc.load_lens();
    if (tid == 0) ticket = lc.claim();
    const int4 c = lc.item(ticket, lane);
    if (tid == 0) claimed[0] = c;
  }
  for (int par = 0;; par ^= 1) {
  // The barrier publishes the item wave 0 resolved and keeps this item's first
  // loads out of LDS the previous item may still be reading.
  lds_barrier();
  const int4 rec = claimed[par];
  const int r = __builtin_amdgcn_readfirstlane(rec.x);
  if (r < 0) break;
  if (tid == 0) ticket = lc.claim();
  const int e0 = __builtin_amdgcn_readfirstlane(rec.y);
  const int e1 = __builtin_amdgcn_readfirstlane(rec.z);
  const int pslot = __builtin_amdgcn_readfirstlane(rec.w);
  const int bh = r / nb, j = r - bh * nb;
  const size_t head = size_t(bh) * size_t(N) * HD;
  const uint32_t hbytes = static_cast<uint32_t>(N) * RB;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(K + head, hbytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(V + head, hbytes);
  const v4i qd = uniform_desc(Q + head, hbytes), dd = uniform_desc(dO + head, hbytes);
  // (LSE log2 e, delta) of the head's rows; rows past N read zeros, which is
  // harmless: their Q and dO rows are zeros too, so they add exactly nothing.
  const v4i ldd = uniform_desc(ld + size_t(bh) * N, static_cast<uint32_t>(N) * 8u);
  const int key = kBB * j + 32 * w + ql;
  const bool key_ok = key < N;
  bf16x8 kf[NDC], vf[NDC];
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    const uint32_t off = uint32_t(key) * RB + uint32_t(32 * c + 16 * hh);
    kf[c] = __builtin_bit_cast(bf16x8, load16(kr, off));
    vf[c] = __builtin_bit_cast(bf16x8, load16(vr, off));
  }
  // Complete these loads before the DMA-pipelined loop.
#pragma unroll
  for (int c = 0; c < NDC; ++c) asm volatile("" ::"v"(kf[c]), "v"(vf[c]));
  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int u = 0; u < NDT; ++u)
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      dk[u][x] = 0.f;
      dv[u][x] = 0.f;
    }
  IndexWindow rows;
  rows.init(row_idx, e0, e1, lane);
  // This wave's halves of query block i into stage st; a block
  // outside [0, nb) reads past the buffers, i.e. zeros.
  auto issue = [&](int i, int st) {
    const bool ok = i >= 0 && i < nb;
    const uint32_t tb = ok ? uint32_t(i) * kTile + uint32_t(w) * kHalf : hbytes;
    const uint32_t sb = lds0 + uint32_t(st) * kStage;
    dma_half_tile<RB>(qd, hoff, tb, sb + uint32_t(w) * kHalf);
    dma_half_tile<RB>(dd, hoff, tb, sb + kTile + uint32_t(w) * kHalf);
    const uint32_t lo = ok ? uint32_t(kBB * i + 32 * w) * 8u + 4u * uint32_t(lane)
                           : static_cast<uint32_t>(N) * 8u;
    dma4(ldd, lo, sb + 2 * kTile + uint32_t(w) * (kLd / 2));
  };
  int i_next = rows.at(e0, lane);
  if (e0 < e1) issue(i_next, 0);
  int pend = 0;  // dS stores issued after the latest tile loads
  for (int e = e0, st = 0; e < e1; ++e, st ^= 1) {
    const int i = i_next;
    // Only block e is in flight (and the dS stores of block e - 1, which are
    // younger): this wave's halves of it have landed once the wait returns.
    // After the barrier both waves' halves are in LDS and both waves are done
    // reading block e-1, whose stage then takes block e+1.
    wait_vm_n(pend);
    pend = 0;
    lds_barrier();
    if (e + 1 < e1) {
      i_next = rows.at(e + 1, lane);
      issue(i_next, st ^ 1);
    } else if (tid < 64) {
      nxt = lc.item(ticket, lane);  // the claim returned by the wait above
    }
    if (i < 0 || i >= nb) continue;
    const uint32_t qs = lds0 + uint32_t(st) * kStage, dss = qs + kTile;
    const float* lds_ld = reinterpret_cast<const float*>(smem + size_t(st) * kStage + 2 * kTile);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const f32x16 zero = {};
      f32x16 s, dp;
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        const bf16x8 qa = lds_read16(qs + swz<RB>(32 * g + ql, 2 * c + hh));
        const bf16x8 da = lds_read16(dss + swz<RB>(32 * g + ql, 2 * c + hh));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[c], c == 0 ? zero : s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[c], c == 0 ? zero : dp, 0, 0, 0);
      }
      // register e of this lane: query 32g + 8(e/4) + 4hh + e%4, key `key`
      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        // (LSE, delta) of queries 32g + 8m + 4hh .. +3, interleaved
        const f32x4 x01 = *reinterpret_cast<const f32x4*>(lds_ld + 2 * (32 * g + 8 * m + 4 * hh));
        const f32x4 x23 = *reinterpret_cast<const f32x4*>(lds_ld + 2 * (32 * g + 8 * m + 4 * hh) + 4);
        const f32x4 L = {x01[0], x01[2], x23[0], x23[2]};
        const f32x4 Dl = {x01[1], x01[3], x23[1], x23[3]};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int ei = 4 * m + x;
          float p = __builtin_amdgcn_exp2f(fmaf(s[ei], c2, -L[x]));
          // Without STORE a key past N reaches only its own column of dK and dV,
          // which is never written out; with STORE its dS enters the tile.
          if constexpr (STORE) p = key_ok ? p : 0.f;
          pb[ei >> 3][ei & 7] = static_cast<__bf16>(p);
          sb[ei >> 3][ei & 7] = static_cast<__bf16>(p * (dp[ei] - Dl[x]));
        }
      }
      // With STORE: dS of this wave's keys for query group g into the pair's tile
      // (slot e) for dq_stored_kernel.  Tile layout: four 2-KiB parts, one per 16 queries
      // (part 2g + k2 holds queries 32g + 16k2 .. +15), each 64 keys x 16
      // queries, key-major.  Elements 0..3 of sb[k2] are queries
      // 32g + 16k2 + 4hh .. +3 and 4..7 those + 8; one swap with the other
      // half-wave gives lane (key, hh) the 8 queries 32g + 16k2 + 8hh .. +7,
      // so each store writes 1 KiB contiguous.
      if constexpr (STORE) {
        uint16_t* dtile = dst_tiles + size_t(e) * (kBB * kBB);
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const uint4 x = __builtin_bit_cast(uint4, sb[k2]);
          const auto s0 = __builtin_amdgcn_permlane32_swap(x.x, x.z, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(x.y, x.w, false, false);
          uint16_t* dst = dtile + size_t((2 * g + k2) * kBB + 32 * w + ql) * 16 + 8 * hh;
          // Non-temporal: the tile is read once, by dq_stored_kernel.
          __builtin_nontemporal_store(v4u{s0[0], s1[0], s0[1], s1[1]}, reinterpret_cast<v4u*>(dst));
        }
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int u = 0; u < NDT; ++u) {
          const int col = 32 * u + tr_col;
          const int r_lo = 32 * g + 16 * k2 + tr_row;
          const uint32_t clo = (col & 7) * 2;
          const v4s dlo = lds_read_tr(dss + swz<RB>(r_lo, col >> 3) + clo);
          const v4s dhi = lds_read_tr(dss + swz<RB>(r_lo + 8, col >> 3) + clo);
          const v4s qlo = lds_read_tr(qs + swz<RB>(r_lo, col >> 3) + clo);
          const v4s qhi = lds_read_tr(qs + swz<RB>(r_lo + 8, col >> 3) + clo);
          const bf16x8 ad = __builtin_bit_cast(bf16x8, __builtin_shufflevector(dlo, dhi, 0, 1, 2, 3, 4, 5, 6, 7));
          const bf16x8 aq = __builtin_bit_cast(bf16x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
          dv[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, pb[k2], dv[u], 0, 0, 0);
          dk[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, sb[k2], dk[u], 0, 0, 0);
        }
    }
    if constexpr (STORE) pend = 4;  // the dS stores above: 2 groups x 2 halves
  }
  // register e of dv[u], dk[u]: dimension 32u + 8(e/4) + 4hh + e%4 of key `key`
  if (pslot >= 0) {
    // [dK | dV] of the block's 64 keys, row-major, fp32; rows of keys past N are never read
    float* pk = part + size_t(pslot) * (2 * kBB * HD) + size_t(32 * w + ql) * HD;
    float* pv = pk + kBB * HD;
#pragma unroll
    for (int u = 0; u < NDT; ++u)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * u + 8 * g4 + 4 * hh;
        *reinterpret_cast<f32x4*>(pk + d) =
            f32x4{dk[u][4 * g4], dk[u][4 * g4 + 1], dk[u][4 * g4 + 2], dk[u][4 * g4 + 3]};
        *reinterpret_cast<f32x4*>(pv + d) =
            f32x4{dv[u][4 * g4], dv[u][4 * g4 + 1], dv[u][4 * g4 + 2], dv[u][4 * g4 + 3]};
      }
  } else if (key_ok) {
    uint16_t* vrow = dV + head + size_t(key) * HD;
    uint16_t* krow = dK + head + size_t(key) * HD;
#pragma unroll
    for (int u = 0; u < NDT; ++u)
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
  if (tid < 64) {
    const int4 c = e1 > e0 ? nxt : lc.item(ticket, lane);
    if (tid == 0) claimed[par ^ 1] = c;
  }
  }
}

// dQ of one chunk of query block i's row (item (bh, i, chunk), two
// wavefronts; wave kh owns keys 32kh .. 32kh+31 of every key block of the row).  The forward's orientation:
// S^T = K Q^T and dP^T = V dO^T with the queries as columns (Q^T, dO^T B
// operands held in registers, one LSE and delta per lane), dS^T = P^T (dP^T -
// delta), and dQ^T += K^T dS^T with K^T read transposed from the wave's LDS
// area.  The two key halves are summed through LDS at the end; an unsplit row
// writes bf16 dQ, a chunk of a split one its fp32 sum (unscaled) to the item's
// partial slot.  At HD = 128 the rings take 64 KiB and the registers
// exceed half the file: one wave per SIMD.
template <int HD>
struct DqCfg {
  static constexpr int RB = HD * 2;
  static constexpr uint32_t kHalf = 32 * RB, kStage = 2 * kHalf;
  static constexpr size_t kClaimAt = 2 * size_t(kDqStages) * kStage;  // two records: the claimed items
  static constexpr size_t LDS_BYTES = kClaimAt + 32;
};

template <int HD>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(HD == 64 ? 2 : 1))) void dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float2* __restrict__ ld,
    const int32_t* __restrict__ col_idx, const int4* __restrict__ items, int32_t* __restrict__ ctr, int32_t n_lists, int32_t list_cap,
    int32_t N, int32_t nb, float c2, float scale, uint16_t* __restrict__ dQ,
    float* __restrict__ part) {
  // Per wave: a ring of kDqStages stages of its 32 key rows of K and of V,
  // streamed by LDS DMA kDqStages - 1 key blocks ahead; no barrier in the loop.
  using C = DqCfg<HD>;
  constexpr int RB = C::RB, NDC = HD / 16, NDT = HD / 32;
  constexpr uint32_t kHalf = C::kHalf, kStage = C::kStage;
  constexpr int kLoads = 2 * (RB / 32);  // tile loads one stage takes per wave
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((BSA_LDS uint8_t*)smem));
  const int lane = threadIdx.x & 63;
  const int kh = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ql = lane & 31, hh = lane >> 5;
  const uint32_t ring = lds0 + uint32_t(kh) * (kDqStages * kStage);
  uint32_t hoff[RB / 32];
  half_offsets<RB>(lane, 32 * kh, hoff);
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  ListClaims lc{items, ctr + kLenQ, ctr + kClaimQ, n_lists, list_cap,
                static_cast<int>(blockIdx.x % n_lists), 0, 0};
  int4* const claimed = reinterpret_cast<int4*>(smem + C::kClaimAt);
  int ticket = 0;
  int4 nxt = make_int4(-1, 0, 0, -1);  // wave 0: the next item, loaded in the last step
  if (threadIdx.x < 64) {
    lc.load_lens();
    if (threadIdx.x == 0) ticket = lc.claim();
    const int4 c = lc.item(ticket, lane);
    if (threadIdx.x == 0) claimed[0] = c;
  }
  for (int par = 0;; par ^= 1) {
  // The barrier publishes the item wave 0 resolved and keeps this item's first
  // loads out of the rings the previous item's key-half exchange may still read.
  lds_barrier();
  const int4 rec = claimed[par];
  const int r = __builtin_amdgcn_readfirstlane(rec.x);
  if (r < 0) break;
  if (threadIdx.x == 0) ticket = lc.claim();
  const int e0 = __builtin_amdgcn_readfirstlane(rec.y);
  const int e1 = __builtin_amdgcn_readfirstlane(rec.z);
  const int pslot = __builtin_amdgcn_readfirstlane(rec.w);
  const int bh = r / nb, i = r - bh * nb;
  const size_t head = size_t(bh) * size_t(N) * HD;
  const uint32_t hbytes = static_cast<uint32_t>(N) * RB;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q + head, hbytes);
  const __amdgpu_buffer_rsrc_t dr = make_rsrc(dO + head, hbytes);
  const v4i kd = uniform_desc(K + head, hbytes), vd = uniform_desc(V + head, hbytes);
  bf16x8 qf[2][NDC], df[2][NDC];
  float L[2], Dl[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int t = kBB * i + 32 * g + ql;
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      const uint32_t off = uint32_t(t) * RB + uint32_t(32 * c + 16 * hh);
      qf[g][c] = __builtin_bit_cast(bf16x8, load16(qr, off));
      df[g][c] = __builtin_bit_cast(bf16x8, load16(dr, off));
    }
    const float2 x = t < N ? ld[size_t(bh) * N + t] : make_float2(INFINITY, 0.f);
    L[g] = x.x;
    Dl[g] = x.y;
  }
  // Complete these loads before the DMA-pipelined loop (a load the compiler sees
  // pending into the loop would make it wait for every DMA at each step).
#pragma unroll
  for (int g = 0; g < 2; ++g) {
#pragma unroll
    for (int c = 0; c < NDC; ++c) asm volatile("" ::"v"(qf[g][c]), "v"(df[g][c]));
    asm volatile("" ::"v"(L[g]), "v"(Dl[g]));
  }
  f32x16 acc[2][NDT];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int u = 0; u < NDT; ++u)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[g][u][x] = 0.f;
  IndexWindow cols;
  cols.init(col_idx, e0, e1, lane);
  // This wave's half of key block j (K, then V) into ring stage st; a column
  // outside [0, nb) reads past the buffers, i.e. zeros.
  auto issue = [&](int j, int st) {
    const bool ok = j >= 0 && j < nb;
    const uint32_t tb = ok ? uint32_t(j) * (kBB * RB) + uint32_t(kh) * kHalf : hbytes;
    const uint32_t dst = ring + uint32_t(st) * kStage;
    dma_half_tile<RB>(kd, hoff, tb, dst);
    dma_half_tile<RB>(vd, hoff, tb, dst + kHalf);
  };
  // Blocks e0 .. e0 + kDqStages - 2 go first; at step e, block e + kDqStages - 1
  // goes into the stage block e - 1 used (its reads are complete), then the
  // wait leaves the younger blocks (kLoads loads each) in flight.
  int jq[kDqStages];
#pragma unroll
  for (int x = 0; x < kDqStages - 1; ++x) {
    jq[x] = cols.at(e0 + x, lane);
    if (e0 + x < e1) issue(jq[x], x);
  }
  for (int e = e0, st = 0; e < e1; ++e, st = st + 1 == kDqStages ? 0 : st + 1) {
    const int ahead = e + kDqStages - 1;
    const int sa = st == 0 ? kDqStages - 1 : st - 1;
    int j = -1;
#pragma unroll
    for (int x = 0; x < kDqStages; ++x)
      if (x == st) j = jq[x];
    if (ahead < e1) {
      const int ja = cols.at(ahead, lane);
#pragma unroll
      for (int x = 0; x < kDqStages; ++x)
        if (x == sa) jq[x] = ja;
      issue(ja, sa);
    }
    wait_vm_n(kLoads * (min(ahead, e1 - 1) - e));
    if (e + 1 == e1 && threadIdx.x < 64) nxt = lc.item(ticket, lane);  // the claim has returned
    if (j < 0 || j >= nb) continue;
    const int kbase = kBB * j + 32 * kh;  // first key of this wave's half
    const uint32_t ks = ring + uint32_t(st) * kStage, vs = ks + kHalf;
    bf16x8 va[NDC], ka[NDC];
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      va[c] = lds_read16(vs + swz<RB>(ql, 2 * c + hh));
      ka[c] = lds_read16(ks + swz<RB>(ql, 2 * c + hh));
    }
    bf16x8 sb[2][2];
    // register x of this lane: key kbase + 8(x/4) + 4hh + x%4, query 32g + ql.
    // Keys past N (only in the last block of a ragged head) get probability 0;
    // the tile body is instantiated twice so that full tiles skip the mask.
    auto tile = [&](auto masked) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const f32x16 zero = {};
        f32x16 s, dp;
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qf[g][c], c == 0 ? zero : s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[c], df[g][c], c == 0 ? zero : dp, 0, 0, 0);
        }
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          float p = __builtin_amdgcn_exp2f(fmaf(s[x], c2, -L[g]));
          if constexpr (decltype(masked)::value) {
            const int kv = kbase + 8 * (x >> 2) + 4 * hh + (x & 3);
            p = kv < N ? p : 0.f;
          }
          sb[g][x >> 3][x & 7] = static_cast<__bf16>(p * (dp[x] - Dl[g]));
        }
      }
    };
    if (kbase + 32 <= N) {
      tile(std::false_type{});
    } else {
      asm volatile("");  // a side effect keeps this a branch, not a select per element
      tile(std::true_type{});
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int u = 0; u < NDT; ++u) {
        const int col = 32 * u + tr_col;
        const uint32_t clo = (col & 7) * 2;
        const v4s lo = lds_read_tr(ks + swz<RB>(16 * k2 + tr_row, col >> 3) + clo);
        const v4s hi = lds_read_tr(ks + swz<RB>(16 * k2 + 8 + tr_row, col >> 3) + clo);
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int g = 0; g < 2; ++g)
          acc[g][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sb[g][k2], acc[g][u], 0, 0, 0);
      }
  }
  // Key-half sum: wave kh finishes query group kh and hands group 1 - kh over.
  // Exchange through the rings (each wave's own is free once its loop ends).
  float* xo = reinterpret_cast<float*>(smem);
  auto send = [&](const f32x16 (&a)[NDT]) {
    float* dst = xo + size_t(kh) * (kDqStages * kStage / 4);
#pragma unroll
    for (int u = 0; u < NDT; ++u)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<f32x4*>(dst + ((u * 4 + g4) * 64 + lane) * 4) =
            f32x4{a[u][4 * g4], a[u][4 * g4 + 1], a[u][4 * g4 + 2], a[u][4 * g4 + 3]};
  };
  auto finish = [&](const f32x16 (&a)[NDT]) {
    const int t = kBB * i + 32 * kh + ql;
    const float* src = xo + size_t(1 - kh) * (kDqStages * kStage / 4);
    if (pslot >= 0) {
      // dQ of the block's 64 queries, row-major, fp32 (queries past N too)
      float* pq = part + size_t(pslot) * (kBB * HD) + size_t(32 * kh + ql) * HD;
#pragma unroll
      for (int u = 0; u < NDT; ++u)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 o1 = *reinterpret_cast<const f32x4*>(src + ((u * 4 + g4) * 64 + lane) * 4);
          const int d = 32 * u + 8 * g4 + 4 * hh;
          *reinterpret_cast<f32x4*>(pq + d) =
              f32x4{a[u][4 * g4] + o1[0], a[u][4 * g4 + 1] + o1[1], a[u][4 * g4 + 2] + o1[2],
                    a[u][4 * g4 + 3] + o1[3]};
        }
      return;
    }
    if (t >= N) return;
    uint16_t* qrow = dQ + head + size_t(t) * HD;
#pragma unroll
    for (int u = 0; u < NDT; ++u)
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
  lds_barrier();
  if (kh == 0)
    finish(acc[0]);
  else
    finish(acc[1]);
  if (threadIdx.x < 64) {
    const int4 c = e1 > e0 ? nxt : lc.item(ticket, lane);
    if (threadIdx.x == 0) claimed[par ^ 1] = c;
  }
  }
}

// dQ from stored dS (head dim 128): the items, key halves, ring and epilogue of
// dq_kernel, but dQ^T += K^T dS^T reads the dS tiles the dK/dV kernel stored
// instead of recomputing S, dP and the exponentials.  Each wave streams its 32
// key rows of K and its 32 keys of the pair's dS tile (4 KiB: 1 KiB of each of
// the tile's four 16-query parts) into its own two-stage LDS ring; K^T and dS^T
// are both read transposed with the same lane pattern, so the keys of the A and
// B operands come in the same order.  At head dim 128 this saves half of the
// kernel's matrix work and all of its exponentials for 16 KiB of memory traffic
// per block pair (measured: 4-8 % faster backward); at head dim 64 the dS
// stream costs more than the recompute (t2i 237 -> 272 us), so dq_kernel stays.
template <int HD>
struct DqsCfg {
  static constexpr int RB = HD * 2;
  static constexpr uint32_t kHalf = 32 * RB;               // the wave's K rows
  static constexpr uint32_t kDsHalf = 32 * kBB * 2;        // its keys of the dS tile
  static constexpr uint32_t kStage = kHalf + kDsHalf;
  static constexpr size_t kClaimAt = 2 * size_t(kDqStages) * kStage;  // two records: the claimed items
  static constexpr size_t LDS_BYTES = kClaimAt + 32;
};

template <int HD>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void dq_stored_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ ds_tiles,
    const int32_t* __restrict__ col_idx, const int32_t* __restrict__ tpos,
    const int4* __restrict__ items, int32_t* __restrict__ ctr, int32_t n_lists, int32_t list_cap,
    int32_t N, int32_t nb, float scale, uint16_t* __restrict__ dQ, float* __restrict__ part) {
  using C = DqsCfg<HD>;
  constexpr int RB = C::RB, NDT = HD / 32;
  constexpr uint32_t kHalf = C::kHalf, kStage = C::kStage;
  constexpr int kLoads = RB / 32 + 4;  // tile loads one stage takes per wave
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((BSA_LDS uint8_t*)smem));
  const int lane = threadIdx.x & 63;
  const int kh = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ql = lane & 31, hh = lane >> 5;
  const uint32_t ring = lds0 + uint32_t(kh) * (kDqStages * kStage);
  uint32_t hoff[RB / 32];
  half_offsets<RB>(lane, 32 * kh, hoff);
  // dS: this wave's 1 KiB of part s sits at 2048 s + 1024 kh in the tile; the
  // loads' immediate offsets add 1024 s to source and destination alike.
  const uint32_t dsrc = uint32_t(1024 * kh + 16 * lane);
  // Lane address of the transposing dS^T reads within a stage's dS area: part
  // 2g + (lane / 16) % 2, key row 16k2 + tr_row, queries 4 (lane % 4) .. +3.
  const uint32_t ds_lane = uint32_t(1024 * ((lane >> 4) & 1) + 32 * (4 * hh + ((lane & 15) >> 2)) +
                                    8 * (lane & 3));
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  ListClaims lc{items, ctr + kLenQ, ctr + kClaimQ, n_lists, list_cap,
                static_cast<int>(blockIdx.x % n_lists), 0, 0};
  int4* const claimed = reinterpret_cast<int4*>(smem + C::kClaimAt);
  int ticket = 0;
  int4 nxt = make_int4(-1, 0, 0, -1);  // wave 0: the next item, loaded in the last step
  if (threadIdx.x < 64) {
    lc.load_lens();
    if (threadIdx.x == 0) ticket = lc.claim();
    const int4 c = lc.item(ticket, lane);
    if (threadIdx.x == 0) claimed[0] = c;
  }
  for (int par = 0;; par ^= 1) {
  // The barrier publishes the item wave 0 resolved and keeps this item's first
  // loads out of the rings the previous item's key-half exchange may still read.
  lds_barrier();
  const int4 rec = claimed[par];
  const int r = __builtin_amdgcn_readfirstlane(rec.x);
  if (r < 0) break;
  if (threadIdx.x == 0) ticket = lc.claim();
  const int e0 = __builtin_amdgcn_readfirstlane(rec.y);
  const int e1 = __builtin_amdgcn_readfirstlane(rec.z);
  const int pslot = __builtin_amdgcn_readfirstlane(rec.w);
  const int bh = r / nb, i = r - bh * nb;
  const size_t head = size_t(bh) * size_t(N) * HD;
  const uint32_t hbytes = static_cast<uint32_t>(N) * RB;
  const v4i kd = uniform_desc(K + head, hbytes);
  f32x16 acc[2][NDT];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int u = 0; u < NDT; ++u)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[g][u][x] = 0.f;
  IndexWindow cols, tiles;
  cols.init(col_idx, e0, e1, lane);
  tiles.init(tpos, e0, e1, lane);
  // This wave's half of key block j's K rows and of the pair's dS^T tile (slot
  // t) into ring stage st; a column outside [0, nb) reads zeros.
  auto issue = [&](int j, int t, int st) {
    const bool ok = j >= 0 && j < nb && t >= 0;
    const uint32_t tb = ok ? uint32_t(j) * (kBB * RB) + uint32_t(kh) * kHalf : hbytes;
    const uint32_t dst = ring + uint32_t(st) * kStage;
    dma_half_tile<RB>(kd, hoff, tb, dst);
    const v4i dd = uniform_desc(ds_tiles + size_t(ok ? t : 0) * (kBB * kBB), ok ? 8192u : 0u);
    dma16x4<true>(dd, dsrc, dsrc + 1024u, dsrc + 2048u, dsrc + 3072u, dst + kHalf);  // read once
  };
  // Blocks e0 .. e0 + kDqStages - 2 go first; at step e, block e + kDqStages - 1
  // goes into the stage block e - 1 used (its reads are complete), then the
  // wait leaves the younger blocks (kLoads loads each) in flight.
  int jq[kDqStages];
#pragma unroll
  for (int x = 0; x < kDqStages - 1; ++x) {
    jq[x] = cols.at(e0 + x, lane);
    const int tq = tiles.at(e0 + x, lane);
    if (e0 + x < e1) issue(jq[x], tq, x);
  }
  for (int e = e0, st = 0; e < e1; ++e, st = st + 1 == kDqStages ? 0 : st + 1) {
    const int ahead = e + kDqStages - 1;
    const int sa = st == 0 ? kDqStages - 1 : st - 1;
    int j = -1;
#pragma unroll
    for (int x = 0; x < kDqStages; ++x)
      if (x == st) j = jq[x];
    if (ahead < e1) {
      const int ja = cols.at(ahead, lane);
      const int ta = tiles.at(ahead, lane);
#pragma unroll
      for (int x = 0; x < kDqStages; ++x)
        if (x == sa) jq[x] = ja;
      issue(ja, ta, sa);
    }
    wait_vm_n(kLoads * (min(ahead, e1 - 1) - e));
    if (e + 1 == e1 && threadIdx.x < 64) nxt = lc.item(ticket, lane);  // the claim has returned
    if (j < 0 || j >= nb) continue;
    const uint32_t ks = ring + uint32_t(st) * kStage, dss = ks + kHalf;
    // dS^T operands: lane (ql, hh) holds query 32g + ql and the keys of the K^T
    // operands below (the same transposing read pattern over key rows).
    bf16x8 sb[2][2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const uint32_t at = dss + uint32_t(2048 * g + 512 * k2) + ds_lane;
        const v4s lo = lds_read_tr(at);
        const v4s hi = lds_read_tr(at + 256u);
        sb[g][k2] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int u = 0; u < NDT; ++u) {
        const int col = 32 * u + tr_col;
        const uint32_t clo = (col & 7) * 2;
        const v4s lo = lds_read_tr(ks + swz<RB>(16 * k2 + tr_row, col >> 3) + clo);
        const v4s hi = lds_read_tr(ks + swz<RB>(16 * k2 + 8 + tr_row, col >> 3) + clo);
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int g = 0; g < 2; ++g)
          acc[g][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sb[g][k2], acc[g][u], 0, 0, 0);
      }
  }
  // Key-half sum: wave kh finishes query group kh and hands group 1 - kh over.
  // Exchange through the rings (each wave's own is free once its loop ends).
  float* xo = reinterpret_cast<float*>(smem);
  auto send = [&](const f32x16 (&a)[NDT]) {
    float* dst = xo + size_t(kh) * (kDqStages * kStage / 4);
#pragma unroll
    for (int u = 0; u < NDT; ++u)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<f32x4*>(dst + ((u * 4 + g4) * 64 + lane) * 4) =
            f32x4{a[u][4 * g4], a[u][4 * g4 + 1], a[u][4 * g4 + 2], a[u][4 * g4 + 3]};
  };
  auto finish = [&](const f32x16 (&a)[NDT]) {
    const int t = kBB * i + 32 * kh + ql;
    const float* src = xo + size_t(1 - kh) * (kDqStages * kStage / 4);
    if (pslot >= 0) {
      // dQ of the block's 64 queries, row-major, fp32 (queries past N too)
      float* pq = part + size_t(pslot) * (kBB * HD) + size_t(32 * kh + ql) * HD;
#pragma unroll
      for (int u = 0; u < NDT; ++u)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 o1 = *reinterpret_cast<const f32x4*>(src + ((u * 4 + g4) * 64 + lane) * 4);
          const int d = 32 * u + 8 * g4 + 4 * hh;
          *reinterpret_cast<f32x4*>(pq + d) =
              f32x4{a[u][4 * g4] + o1[0], a[u][4 * g4 + 1] + o1[1], a[u][4 * g4 + 2] + o1[2],
                    a[u][4 * g4 + 3] + o1[3]};
        }
      return;
    }
    if (t >= N) return;
    uint16_t* qrow = dQ + head + size_t(t) * HD;
#pragma unroll
    for (int u = 0; u < NDT; ++u)
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
  lds_barrier();
  if (kh == 0)
    finish(acc[0]);
  else
    finish(acc[1]);
  if (threadIdx.x < 64) {
    const int4 c = e1 > e0 ? nxt : lc.item(ticket, lane);
    if (threadIdx.x == 0) claimed[par ^ 1] = c;
  }
  }
}

// The split blocks: the chunks' fp32 partials summed in chunk order, then bf16
// dK (times scale) and dV of key column r, and dQ (times scale) of CSR row r
// (r = bh nb + block).  Rows past N are not stored.  Unsplit blocks were
// written by the gradient kernels.
template <int HD>
__global__ __launch_bounds__(256) void reduce_kernel(const int2* __restrict__ col_split,
                                                     const int2* __restrict__ row_split,
                                                     const float* __restrict__ part_kv,
                                                     const float* __restrict__ part_q, int32_t N,
                                                     int32_t nb, float scale,
                                                     uint16_t* __restrict__ dK,
                                                     uint16_t* __restrict__ dV,
                                                     uint16_t* __restrict__ dQ) {
  const int r = blockIdx.x;
  const int bh = r / nb, blk = r - bh * nb;
  const size_t head = size_t(bh) * size_t(N) * HD;
  const int tid = threadIdx.x;
  constexpr int kIters = kBB * HD / 4 / 256;
  auto store4 = [&](uint16_t* T, int e, f32x4 x, float f) {
    const int t = kBB * blk + e / HD;
    if (t >= N) return;
    *reinterpret_cast<uint2*>(T + head + size_t(t) * HD + (e % HD)) =
        make_uint2(pack_bf16x2(f * x[0], f * x[1]), pack_bf16x2(f * x[2], f * x[3]));
  };
  const int2 sk = col_split[r];
  if (sk.x >= 0 && sk.y > 1) {
#pragma unroll
    for (int x = 0; x < kIters; ++x) {
      const int e = 4 * (tid + 256 * x);  // element of the 64 x HD block
      f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
      for (int c = 0; c < sk.y; ++c) {
        const float* p = part_kv + size_t(sk.x + c) * (2 * kBB * HD);
        a += *reinterpret_cast<const f32x4*>(p + e);
        b += *reinterpret_cast<const f32x4*>(p + kBB * HD + e);
      }
      store4(dK, e, a, scale);
      store4(dV, e, b, 1.f);
    }
  }
  const int2 sq = row_split[r];
  if (sq.x >= 0 && sq.y > 1) {
#pragma unroll
    for (int x = 0; x < kIters; ++x) {
      const int e = 4 * (tid + 256 * x);
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
      for (int c = 0; c < sq.y; ++c)
        a += *reinterpret_cast<const f32x4*>(part_q + size_t(sq.x + c) * (kBB * HD) + e);
      store4(dQ, e, a, scale);
    }
  }
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Chunk length of the split: twice the mean CSR row length, at least 16.
int32_t chunk_len(int64_t nnz, int64_t n_rows) {
  const int64_t mean = n_rows > 0 ? (nnz + n_rows - 1) / n_rows : 0;
  return static_cast<int32_t>(std::max<int64_t>(16, std::min<int64_t>(2 * mean, 1 << 20)));
}

// Partial slots for each of the two split kinds: a split block of L > chunk
// entries takes ceil(L / chunk) < 2 L / chunk slots, and the blocks of each
// kind partition at most nnz entries.
int64_t slot_cap(int64_t nnz, int32_t chunk) { return 2 * nnz / chunk + 1; }

// Chunks a split column or row is cut into at most.
int32_t max_chunks(int32_t nb, int32_t chunk) { return std::max(1, (nb + chunk - 1) / chunk); }

// Work lists of the gradient kernels and the records each holds at most: every
// head of a list contributes at most nb max_ch items.
int32_t n_work_lists(int32_t n_heads) { return n_heads >= kLists ? kLists : 1; }
int64_t list_cap(int32_t n_heads, int32_t nb, int32_t max_ch) {
  const int32_t nl = n_work_lists(n_heads);
  return int64_t((n_heads + nl - 1) / nl) * nb * max_ch;
}

struct BwdLayout {
  size_t ld, col_ptr, row_idx, col_split, row_split, ctr, items_kv, items_q, tpos, ds, part_kv,
      part_q, total;
};

BwdLayout bwd_layout(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, int64_t nnz) {
  BwdLayout L{};
  const size_t rows = size_t(B) * H * N;
  const int32_t nb = n_blocks(N, block);
  const size_t nrow = size_t(B) * H * nb;
  const int32_t chunk = chunk_len(nnz, int64_t(nrow));
  const int64_t cap = slot_cap(nnz, chunk);
  const size_t lists = 2 * size_t(n_work_lists(B * H)) * list_cap(B * H, nb, max_chunks(nb, chunk));
  size_t o = 0;
  L.ld = o;        o += round256(rows * sizeof(float2));
  L.col_ptr = o;   o += round256((nrow + 1) * sizeof(int32_t));
  L.row_idx = o;   o += round256(size_t(nnz) * sizeof(int32_t));
  L.col_split = o; o += round256(nrow * sizeof(int2));
  L.row_split = o; o += round256(nrow * sizeof(int2));
  L.ctr = o;       o += round256(kCtrInts * sizeof(int32_t));
  L.items_kv = o;  o += round256(lists * sizeof(int4));
  L.items_q = o;   o += round256(lists * sizeof(int4));
  const size_t stored = D == 128 ? size_t(nnz) : 0;  // dS tiles kept at head dim 128
  L.tpos = o;      o += round256(stored * sizeof(int32_t));
  L.ds = o;        o += stored * kBB * kBB * sizeof(uint16_t);
  L.part_kv = o;   o += round256(size_t(cap) * 2 * kBB * size_t(D) * sizeof(float));
  L.part_q = o;    o += round256(size_t(cap) * kBB * size_t(D) * sizeof(float));
  L.total = o;
  return L;
}

// A 128-block CSR as the 64-block CSR of the same mask: query block i of 128
// rows is query blocks 2i and 2i + 1 of 64 rows (the second only if it starts
// before N), key block j is key blocks 2j and 2j + 1.  CSR row r = bh nb128 + i
// owns entries [4 rp[r], 4 rp[r + 1]) of the result: the first half for row
// 2i of head bh, the second for row 2i + 1, whose columns are (2j, 2j + 1) for
// every listed j in order; when row 2i + 1 does not exist, row 2i's range also
// takes the second half, filled with -1 (a column the backward ignores), and
// so does a column 2j + 1 past the last 64-block.  One workgroup per row.
__global__ __launch_bounds__(64) void refine_kernel(const int32_t* __restrict__ rp,
                                                   const int32_t* __restrict__ ci, int32_t nb128,
                                                   int32_t nb64, int32_t n_rows,
                                                   int32_t* __restrict__ rp64,
                                                   int32_t* __restrict__ ci64) {
  const int r = blockIdx.x;
  const int bh = r / nb128, i = r - bh * nb128;
  const int b = rp[r], len = rp[r + 1] - b;
  const bool second = 2 * i + 1 < nb64;
  const int r64 = bh * nb64 + 2 * i;
  if (threadIdx.x == 0) {
    rp64[r64] = 4 * b;
    if (second) rp64[r64 + 1] = 4 * b + 2 * len;
    if (r == n_rows - 1) rp64[bh * nb64 + nb64] = 4 * rp[n_rows];
  }
  for (int m = threadIdx.x; m < len; m += 64) {
    const int j = ci[b + m];
    const int c0 = 2 * j, c1 = (j >= 0 && 2 * j + 1 < nb64) ? 2 * j + 1 : -1;
    ci64[4 * b + 2 * m] = c0;
    ci64[4 * b + 2 * m + 1] = c1;
    ci64[4 * b + 2 * len + 2 * m] = second ? c0 : -1;
    ci64[4 * b + 2 * len + 2 * m + 1] = second ? c1 : -1;
  }
}

// dS tiles are stored by the dK/dV kernel and read by dq_stored_kernel at head
// dim 128; at head dim 64 dq_kernel recomputes them.
template <int HD>
constexpr bool kStoreDs = HD == 128;

template <int HD>
const void* dkdv_fn() {
  return reinterpret_cast<const void*>(&dkdv_kernel<HD, kStoreDs<HD>>);
}
template <int HD>
const void* dq_fn() {
  if constexpr (kStoreDs<HD>) return reinterpret_cast<const void*>(&dq_stored_kernel<HD>);
  return reinterpret_cast<const void*>(&dq_kernel<HD>);
}
template <int HD>
constexpr size_t dq_lds() {
  return kStoreDs<HD> ? DqsCfg<HD>::LDS_BYTES : DqCfg<HD>::LDS_BYTES;
}

// Resident workgroups of the dK/dV (KV) or dQ kernel on the current device
// (cached; the kernels' LDS attributes are set before the first call).
template <int HD, bool KV>
int resident_grad_workgroups() {
  static std::once_flag once;
  static int n = 0;
  std::call_once(once, [] {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return;
    const void* f = KV ? dkdv_fn<HD>() : dq_fn<HD>();
    const size_t lds = KV ? DkdvCfg<HD>::LDS_BYTES : dq_lds<HD>();
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, 128, lds) != hipSuccess) return;
    n = cus * (per_cu > 0 ? per_cu : 1);
  });
  return n;
}

// The five launches for head dim HD (see the top of the file).
template <int HD>
bsa_status launch_backward(const void* q, const void* k, const void* v, const void* o,
                           const void* d_o, const float* lse, int32_t B, int32_t H, int32_t N,
                           int32_t block, const int32_t* row_ptr, const int32_t* col_idx,
                           int64_t nnz, float sc, void* dq, void* dk, void* dv, uint8_t* ws,
                           hipStream_t s) {
  const int32_t nb = n_blocks(N, block);
  const int64_t rows = int64_t(B) * H * N;
  const int32_t n_heads = B * H;
  const int32_t n_rows = n_heads * nb;
  const int32_t chunk = chunk_len(nnz, n_rows);
  const int32_t max_ch = max_chunks(nb, chunk);
  const int64_t cap = slot_cap(nnz, chunk);
  const int32_t n_lists = n_work_lists(n_heads);
  const int64_t lcap = list_cap(n_heads, nb, max_ch);
  if (int64_t(n_rows) * max_ch > INT32_MAX || cap > INT32_MAX || 2 * lcap * n_lists > INT32_MAX)
    return BSA_ERR_UNSUPPORTED;
  const BwdLayout lay = bwd_layout(B, H, N, HD, block, nnz);
  float2* ld = reinterpret_cast<float2*>(ws + lay.ld);
  int32_t* col_ptr = reinterpret_cast<int32_t*>(ws + lay.col_ptr);
  int32_t* row_idx = reinterpret_cast<int32_t*>(ws + lay.row_idx);
  int2* col_split = reinterpret_cast<int2*>(ws + lay.col_split);
  int2* row_split = reinterpret_cast<int2*>(ws + lay.row_split);
  int32_t* ctr = reinterpret_cast<int32_t*>(ws + lay.ctr);
  int4* items_kv = reinterpret_cast<int4*>(ws + lay.items_kv);
  int4* items_q = reinterpret_cast<int4*>(ws + lay.items_q);
  int32_t* tpos = reinterpret_cast<int32_t*>(ws + lay.tpos);
  uint16_t* ds = reinterpret_cast<uint16_t*>(ws + lay.ds);
  float* part_kv = reinterpret_cast<float*>(ws + lay.part_kv);
  float* part_q = reinterpret_cast<float*>(ws + lay.part_q);

  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&transpose_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               kMaxBlocks * (kMaxBlocks / 32) * 4);
    if (attr == hipSuccess)
      attr = hipFuncSetAttribute(dkdv_fn<HD>(), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 static_cast<int>(DkdvCfg<HD>::LDS_BYTES));
    if (attr == hipSuccess)
      attr = hipFuncSetAttribute(dq_fn<HD>(), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 static_cast<int>(dq_lds<HD>()));
  });
  if (attr != hipSuccess) return BSA_ERR_HIP;

  constexpr int kLpr = HD / 8;  // prep lanes per row
  hipLaunchKernelGGL(prep_kernel<HD>, dim3(static_cast<uint32_t>((rows * kLpr + 255) / 256)),
                     dim3(256), 0, s, static_cast<const uint16_t*>(o),
                     static_cast<const uint16_t*>(d_o), lse, rows, ld, ctr);
  BSA_HIP_CHECK_LAUNCH();
  const size_t bits_bytes = size_t(nb) * ((nb + 31) / 32) * 4;
  hipLaunchKernelGGL(transpose_kernel, dim3(n_heads), dim3(256), bits_bytes, s, row_ptr, col_idx,
                     nb, n_heads, col_ptr, row_idx, chunk, max_ch, ctr, static_cast<int32_t>(cap),
                     static_cast<int32_t>(cap), col_split, row_split, n_lists,
                     static_cast<int32_t>(lcap), items_kv, items_q);
  BSA_HIP_CHECK_LAUNCH();
  if constexpr (kStoreDs<HD>) {
    hipLaunchKernelGGL(tpos_kernel, dim3(static_cast<uint32_t>(n_rows)), dim3(64), 0, s, row_ptr,
                       col_idx, col_ptr, row_idx, nb, tpos);
    BSA_HIP_CHECK_LAUNCH();
  }
  const float c2 = sc * kLog2e;
  // Persistent grids: the resident workgroups, at most one per possible item.
  const int res_kv = resident_grad_workgroups<HD, true>();
  const int res_q = resident_grad_workgroups<HD, false>();
  if (res_kv <= 0 || res_q <= 0) return BSA_ERR_HIP;
  const int64_t slots = int64_t(n_rows) * max_ch;
  const dim3 grid_kv(static_cast<uint32_t>(std::min<int64_t>(res_kv, slots)));
  const dim3 grid_q(static_cast<uint32_t>(std::min<int64_t>(res_q, slots)));
  hipLaunchKernelGGL((dkdv_kernel<HD, kStoreDs<HD>>), grid_kv, dim3(128), DkdvCfg<HD>::LDS_BYTES, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(d_o), ld,
                     row_idx, items_kv, ctr, n_lists, static_cast<int32_t>(lcap), N, nb, c2, sc,
                     static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), part_kv, ds);
  BSA_HIP_CHECK_LAUNCH();
  if constexpr (kStoreDs<HD>) {
    hipLaunchKernelGGL(dq_stored_kernel<HD>, grid_q, dim3(128), DqsCfg<HD>::LDS_BYTES, s,
                       static_cast<const uint16_t*>(k), ds, col_idx, tpos, items_q, ctr, n_lists,
                       static_cast<int32_t>(lcap), N, nb, sc, static_cast<uint16_t*>(dq), part_q);
  } else {
    hipLaunchKernelGGL(dq_kernel<HD>, grid_q, dim3(128), DqCfg<HD>::LDS_BYTES, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(d_o), ld,
                       col_idx, items_q, ctr, n_lists, static_cast<int32_t>(lcap), N, nb, c2, sc,
                       static_cast<uint16_t*>(dq), part_q);
  }
  BSA_HIP_CHECK_LAUNCH();
  if (max_ch > 1) {
    hipLaunchKernelGGL(reduce_kernel<HD>, dim3(static_cast<uint32_t>(n_rows)), dim3(256), 0, s,
                       col_split, row_split, part_kv, part_q, N, nb, sc,
                       static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv),
                       static_cast<uint16_t*>(dq));
    BSA_HIP_CHECK_LAUNCH();
  }
  return BSA_OK;
}

}  // namespace
}  // namespace bsa

extern "C" BSA_API size_t bsa_backward_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t D,
                                                      int32_t block, int64_t nnz) {
  using namespace bsa;
  if (B < 1 || H < 1 || N < 1 || D < 1 || block < 1 || nnz < 0) return 0;
  if (block != 2 * kBB) return bwd_layout(B, H, N, D, block, nnz).total;
  // Block 128: the 64-block CSR of the same mask first, then the block-64
  // workspace for its (at most 4 nnz) entries.
  const size_t rows64 = size_t(B) * H * n_blocks(N, kBB);
  return round256((rows64 + 1) * sizeof(int32_t)) + round256(size_t(4 * nnz) * sizeof(int32_t)) +
         bwd_layout(B, H, N, D, kBB, 4 * nnz).total;
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
  if ((D != 64 && D != 128) || (block != kBB && block != 2 * kBB)) return BSA_ERR_UNSUPPORTED;
  const int32_t nb = n_blocks(N, kBB);  // 64-row blocks (a block-128 CSR is refined)
  if (nb > kMaxBlocks || int64_t(N) * D * 2 >= (int64_t(1) << 31) || 4 * nnz > INT32_MAX ||
      int64_t(B) * H * nb > INT32_MAX)
    return BSA_ERR_UNSUPPORTED;
  for (const void* p : {q, k, v, o, d_o, static_cast<const void*>(dq), static_cast<const void*>(dk),
                        static_cast<const void*>(dv), static_cast<const void*>(workspace)})
    if (!aligned16(p)) return BSA_ERR_INVALID_ARG;
  if (workspace_bytes < bsa_backward_workspace_bytes(B, H, N, D, block, nnz))
    return BSA_ERR_CAPACITY;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const float sc = scale > 0.f ? scale : 1.f / sqrtf(static_cast<float>(D));
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (block == 2 * kBB) {
    const int32_t nb128 = n_blocks(N, block), rows128 = B * H * nb128;
    int32_t* rp64 = reinterpret_cast<int32_t*>(ws);
    const size_t rp_bytes = round256((size_t(B) * H * nb + 1) * sizeof(int32_t));
    int32_t* ci64 = reinterpret_cast<int32_t*>(ws + rp_bytes);
    hipLaunchKernelGGL(refine_kernel, dim3(static_cast<uint32_t>(rows128)), dim3(64), 0, s,
                       row_ptr, col_idx, nb128, nb, rows128, rp64, ci64);
    BSA_HIP_CHECK_LAUNCH();
    row_ptr = rp64;
    col_idx = ci64;
    nnz *= 4;
    block = kBB;
    ws += rp_bytes + round256(size_t(nnz) * sizeof(int32_t));
  }
  if (D == 64)
    return launch_backward<64>(q, k, v, o, d_o, lse, B, H, N, block, row_ptr, col_idx, nnz, sc,
                               dq, dk, dv, ws, s);
  return launch_backward<128>(q, k, v, o, d_o, lse, B, H, N, block, row_ptr, col_idx, nnz, sc,
                              dq, dk, dv, ws, s);
}
