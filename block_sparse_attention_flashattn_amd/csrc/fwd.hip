// Block-sparse FlashAttention forward for gfx950 (MI355X).
//
// BSA-DiT §4.1: the FlashAttention tile loop keeps its outer loop over query
// blocks, and its inner loop visits only the KV blocks listed for that query
// block in a compact index read from global memory (here CSR).  BSA-DiT §4.3:
// the online softmax is carried over the visited blocks only and divided by
// their true total at the end, which is exactly the softmax with skipped
// blocks at -inf.
//
// Kernel design
//   * Persistent workgroups: workgroup w runs work items w, w + G, w + 2G, ...
//     (G = resident workgroups).  An item is a query block of one head (a CSR
//     row) or a chunk of one.  The tiles of consecutive items form one stream,
//     so the next item's first K/V tiles, its query fragment, metadata and
//     column indices are already in flight while the current item finishes.
//   * 2*BLK/32 wavefronts: BLK/32 query groups of 32 rows times 2 key halves.
//     Wave (g, h) keeps its own online-softmax state for query rows
//     32g..32g+31 over keys h*BLK/2 .. (h+1)*BLK/2-1 of every tile; the halves
//     merge through LDS once per item.
//   * K and V tiles go from HBM straight into an LDS ring (buffer loads with
//     the `lds` bit, 16 bytes per lane, no VGPR staging), NSTAGE-1 tiles ahead
//     of the computation.  Both tiles are row-major with 16-byte chunks XOR-
//     swizzled by row (chunk_swizzle), which keeps the LDS read patterns
//     below free of bank conflicts.  Buffer bounds turn keys past N and invalid columns into
//     zeros without branches.  The wait for a tile is an explicit vmcnt that
//     leaves the younger tiles in flight.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the accumulator of a lane holds
//     16 keys of ONE query, so row max / row sum are in-lane plus one
//     v_permlane32_swap, and P^T leaves the accumulator already in the
//     B-operand layout of the next product.
//   * O^T += V^T P^T on the same MFMA; the V^T operand is read from the
//     row-major V tile with the transposing LDS read ds_read_b64_tr_b16 (two
//     per 16-key step), so V is never transposed in registers.
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
#include "tile.h"
#include "dma.h"

namespace bsa {
namespace {


template <int BLK, int HD>
struct FwdCfg {
  static constexpr int NQG = BLK / 32;              // query groups of 32 rows
  static constexpr int NW = 2 * NQG;                // wavefronts: query group x key half
  static constexpr int NT = 64 * NW;                // threads per workgroup (= 4 * BLK)
  static constexpr int ROWB = HD * 2;               // bytes of one K/V/Q row
  static constexpr int CPR = HD / 8;                // 16-byte chunks per row
  static constexpr int TILEB = BLK * ROWB;          // bytes of one K or V tile
  static constexpr int STAGEB = 2 * TILEB;          // K tile then V tile
  static constexpr int NSTAGE = TILEB <= 8192 ? 3 : 2;
  static constexpr int DPW = STAGEB / 1024 / NW;    // 16-byte-per-lane loads per wave per tile
  static constexpr int ML_FLOATS = NQG * 64 * 2;    // merge area: running max and sum
  static constexpr size_t LDS_BYTES = size_t(NSTAGE) * STAGEB + ML_FLOATS * 4 + 16;
  static constexpr int NDC = HD / 16;               // k-steps of the QK^T product
  static constexpr int NKT = BLK / 64;              // 32-key subtiles per key half
  static constexpr int NDT = HD / 32;               // 32-wide d subtiles of the output
  static_assert(DPW * NW * 1024 == STAGEB, "loads must cover a stage exactly");
  static_assert(size_t(NQG) * 64 * NDT * 16 * 4 <= size_t(STAGEB),
                "the accumulator merge must fit in one stage");
  static_assert(BLK <= 255, "valid counts are queued in 8-bit fields");
};



// Cache policy of buffer accesses shared between workgroups on different dies
// (sc1): coherent at device scope, as the agent-scope atomic accesses are.
constexpr int kAgentScope = 16;


// Uniform load of a read-only table entry through the constant address space:
// the compiler then always uses a scalar load, whatever it can prove about the
// kernel's stores and atomics aliasing the table.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p, size_t i) {
  return reinterpret_cast<const __attribute__((address_space(4))) T*>(
      reinterpret_cast<uintptr_t>(p))[i];
}

// Item counters at the start of the forward workspace (with a work list): one
// per group, each on its own 4-KB page so that claims on different groups do
// not queue behind each other in one memory channel.
constexpr int kCounterStride = 1024;  // int32 entries
constexpr size_t kCounterBytes = size_t(BSA_MAX_GROUPS) * kCounterStride * sizeof(int32_t);
// Merge counters: one int32 per query group of a 64-query block (two) and
// partial slot, rounded up to 256 bytes; they follow the item counters.
inline size_t merge_counter_bytes(int32_t n_slots) {
  return (size_t(n_slots) * 2 * sizeof(int32_t) + 255) & ~size_t(255);
}

// Where a persistent workgroup's items come from.
//  * No work list: workgroup w runs CSR rows w, w + G, w + 2G, ... (static).
//  * Work list: the items come in groups (table after the merge records);
//    workgroup w serves group w % ng, runs its items w / ng and w / ng + Gg
//    (Gg = workgroups of the group) and claims the rest in list order from
//    the group's counter, one item before it needs it.  A workgroup claims
//    while its previous claim (or its second static item) was an item, so the
//    group's claims are the items past the static rounds plus one failed claim
//    per claiming workgroup; whoever receives the last claim number resets
//    the counter for the next call.  Claims are vector atomics from one lane.
struct ItemSource {
  int32_t ng, grp, lw, gx, base, size, total;

  __device__ void init(const int32_t* w, int32_t n_items, int32_t n_merges, int32_t n_rows) {
    const int G = gridDim.x;
    if (w) {
      const int32_t* gt = w + 4 * size_t(n_items) + 3 * size_t(n_merges);
      ng = min(max(ld_uniform(gt, 0), 1), BSA_MAX_GROUPS);
      grp = blockIdx.x % ng;
      lw = blockIdx.x / ng;
      gx = (G - grp + ng - 1) / ng;
      base = min(max(ld_uniform(gt, 1 + grp), 0), n_items);
      size = min(max(ld_uniform(gt, 2 + grp), base), n_items) - base;
    } else {
      ng = 1;
      grp = 0;
      lw = blockIdx.x;
      gx = G;
      base = 0;
      size = n_rows;
    }
    total = max(size - 2 * gx, 0) + min(gx, max(size - gx, 0));
  }
  // Item of static round r of this workgroup, or -1.
  __device__ int stat(int r) const {
    const int64_t p = lw + int64_t(r) * gx;
    return p < size ? base + static_cast<int>(p) : -1;
  }
  // Item won by claim number `ticket` of the group, or -1.
  __device__ int claimed(int ticket) const {
    const int64_t p = 2 * int64_t(gx) + ticket;
    return (ticket >= 0 && p < size) ? base + static_cast<int>(p) : -1;
  }
  // One claim (call from a single lane); the result is the claim number.
  __device__ int claim(int32_t* ctr) const {
    return __hip_atomic_fetch_add(ctr + size_t(grp) * kCounterStride, 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  }
  // After claim number `ticket` returned (single lane): the last claim of the
  // group resets its counter.
  __device__ void retire(int32_t* ctr, int ticket) const {
    if (ticket == total - 1)
      __hip_atomic_store(ctr + size_t(grp) * kCounterStride, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
};

// Largest growth of the running max (log2 units) tolerated before the
// accumulator is rescaled; probabilities then stay below 2^8 before the final
// division, well inside fp32 and bf16 range.
constexpr float kRescaleSlack = 8.0f;
// Largest lane-partial row sum of one tile's probabilities (each taken against
// the running max as it stands) accepted without raising the max: every such
// probability is then below 2^20, so the accumulators stay far inside fp32
// range and the bf16 operand keeps its relative precision.
constexpr float kSumCap = 1048576.0f;



// RES: O = attention + R (a residual added before O is rounded).
template <int BLK, int HD, bool RES>
__global__ __launch_bounds__(4 * BLK) __attribute__((amdgpu_waves_per_eu(2))) void fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, const int32_t* __restrict__ work, int32_t n_items,
    int32_t n_merges, int32_t N, int32_t nb, int32_t n_rows, float sl2, uint16_t* __restrict__ O,
    float* __restrict__ LSE, float* __restrict__ part, int32_t* __restrict__ ctr,
    const uint16_t* __restrict__ R) {
  using C = FwdCfg<BLK, HD>;
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((BSA_LDS uint8_t*)smem));
  float* ml = reinterpret_cast<float*>(smem + size_t(C::NSTAGE) * C::STAGEB);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  const int qg = wave % C::NQG;  // query group
  const int kh = wave / C::NQG;  // key half
  const int ql = lane & 31;      // query column of this lane in the MFMA tiles
  const int hh = lane >> 5;      // which half of the k / row dimension the lane feeds
  const uint32_t head_bytes = static_cast<uint32_t>(size_t(N) * C::ROWB);
  const int nnz = ld_uniform(row_ptr, n_rows);
  const int32_t* col_src = nnz > 0 ? col_idx : row_ptr;  // valid for index 0

  // Work item k -> (row, first column position, column count, slot); row = -1
  // when k is past the end.  Everything here is wavefront-uniform.
  auto load_item = [&](int k, int& row, int& c0, int& cnt, int& slot) {
    row = -1;
    c0 = cnt = 0;
    slot = -1;
    if (k < 0 || k >= n_items) return;
    int r, b, e, sl;
    if (work) {
      r = ld_uniform(work, 4 * size_t(k));
      b = ld_uniform(work, 4 * size_t(k) + 1);
      e = ld_uniform(work, 4 * size_t(k) + 2);
      sl = ld_uniform(work, 4 * size_t(k) + 3);
    } else {
      r = k;
      b = ld_uniform(row_ptr, k);
      e = ld_uniform(row_ptr, k + 1);
      sl = -1;
    }
    if (r < 0 || r >= n_rows) return;
    b = min(max(b, 0), nnz);
    e = min(max(e, b), nnz);
    row = r;
    c0 = b;
    cnt = e - b;
    slot = sl;
  };

  // This wave's share of a stage: DPW loads of 64 chunks; waves [0, NW/2) fill
  // the K tile, the others the V tile.  Load i brings the chunk that lands at
  // this lane's (swizzled) LDS position of segment i; its source offset lies
  // at least 1024 i bytes into the tile (segment i holds tile rows at or past
  // 1024 i / ROWB), so doff[i] = source offset - 1024 (i % 4) >= 0 serves the
  // four-load groups of dma16x4.
  static_assert(C::DPW % 4 == 0, "loads go in groups of four");
  const bool loads_v = wave >= C::NW / 2;
  uint32_t doff[C::DPW];
#pragma unroll
  for (int i = 0; i < C::DPW; ++i) {
    const int g = (wave * C::DPW + i) * 64 + lane - (loads_v ? BLK * C::CPR : 0);
    const int row = g / C::CPR;
    const int pos = g - row * C::CPR;
    doff[i] = uint32_t(row) * C::ROWB + uint32_t((pos ^ chunk_swizzle<C::ROWB>(row)) << 4) -
              uint32_t(i & 3) * 1024u;
  }

  // This wave's K or V buffer descriptor for the head of CSR row `row`
  // (rows < 0: an empty range).  Built once per item.
  auto kv_desc = [&](int row) -> v4i {
    const int bh = row >= 0 ? row / nb : 0;
    v4i d = make_desc((loads_v ? V : K) + size_t(bh) * size_t(N) * HD, row >= 0 ? head_bytes : 0u);
#pragma unroll
    for (int w = 0; w < 4; ++w) d[w] = __builtin_amdgcn_readfirstlane(d[w]);
    return d;
  };
  const uint32_t lds_wave = lds0 + uint32_t(wave * C::DPW) * 1024u;

  // Issue this wave's loads of tile `j` (through descriptor `desc`) into ring
  // stage `st`.  Out-of-range columns point past the end: zeros.
  auto issue_tile = [&](const v4i& desc, int j, int st) {
    const uint32_t tb = (j >= 0 && j < nb) ? uint32_t(j) * C::TILEB : head_bytes;
    const uint32_t l0 = lds_wave + uint32_t(st) * C::STAGEB;
#pragma unroll
    for (int i = 0; i < C::DPW; i += 4)
      dma16x4(desc, tb + doff[i], tb + doff[i + 1], tb + doff[i + 2], tb + doff[i + 3],
              l0 + uint32_t(i) * 1024u);
  };

  // Query fragment of the item on CSR row `row` (B operand of S^T = K Q^T):
  // lane holds d = 16c + 8hh .. +7 of query row 32*qg + ql.  Rows past N, and
  // every row of an empty item (row < 0), read as zeros.
  auto load_q = [&](int row, bf16x8* qf) {
    const int bh = row >= 0 ? row / nb : 0;
    const int qrow = (row >= 0 ? row - bh * nb : 0) * BLK + qg * 32 + ql;
    const __amdgpu_buffer_rsrc_t qrs =
        make_rsrc(Q + size_t(bh) * size_t(N) * HD, row >= 0 ? head_bytes : 0u);
    const uint32_t qoff = static_cast<uint32_t>(qrow) * C::ROWB;
#pragma unroll
    for (int c = 0; c < C::NDC; ++c)
      qf[c] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff + (2 * c + hh) * 16, 0, 0));
  };

  // ---- item source --------------------------------------------------------
  ItemSource src;
  src.init(work, n_items, n_merges, n_rows);
  const bool queue = work != nullptr;
  int k_cur = src.stat(0), k_nxt = src.stat(1);
  int round = 2;           // static round of the item after next (no work list)
  bool claim_out = false;  // a claim for the item after next is in flight
  int ticket = -1;         // its claim number, in lane 0 of wave 0
  if (k_cur < 0) return;
  claim_out = queue && k_nxt >= 0;
  if (claim_out && wave == 0 && lane == 0) ticket = src.claim(ctr);

  // ---- stream state -------------------------------------------------------
  int cur_row, cur_c0, cur_cnt, cur_slot, nxt_row, nxt_c0, nxt_cnt, nxt_slot;
  load_item(k_cur, cur_row, cur_c0, cur_cnt, cur_slot);
  load_item(k_nxt, nxt_row, nxt_c0, nxt_cnt, nxt_slot);
  v4i desc_cur = kv_desc(cur_row), desc_nxt = kv_desc(nxt_row);
  bf16x8 qf[C::NDC], qn[C::NDC];
  load_q(cur_row, qf);
  load_q(nxt_row, qn);

  // The stream is the current item's tiles followed by the next item's.  With
  // u tiles of the current item computed and `inflight` issued ahead, the next
  // tile to issue is stream tile u + inflight.
  int inflight = 0;  // tiles issued and not yet computed
  int st_next = 0;   // ring stage of the next issued tile
  uint32_t vq = 0;   // valid key counts of the tiles in flight, 8 bits each, oldest lowest
  // Column position of stream tile t (or -1 past the next item), and whether
  // it belongs to the next item.
  auto stream_src = [&](int t, bool& in_next) -> int {
    in_next = t >= cur_cnt;
    const int tn = t - cur_cnt;
    return !in_next ? cur_c0 + t : (tn < nxt_cnt ? nxt_c0 + tn : -1);
  };
  auto issue = [&](int j, bool in_next) {
    issue_tile(in_next ? desc_nxt : desc_cur, j, st_next);
    const uint32_t valid = (j >= 0 && j < nb) ? uint32_t(min(BLK, N - j * BLK)) : 0u;
    vq |= valid << (8 * inflight);
    ++inflight;
    st_next = st_next + 1 == C::NSTAGE ? 0 : st_next + 1;
  };
  // Fill the ring (all but one stage) with the next tiles of the stream; `u`
  // tiles of the current item have been computed.
  auto refill = [&](int u) {
    while (inflight + 1 < C::NSTAGE) {
      bool in_next;
      const int src = stream_src(u + inflight, in_next);
      if (src < 0) break;
      issue(ld_uniform(col_idx, src), in_next);
    }
  };

  // Retire the query loads before any tile load is issued, so that the wait
  // bookkeeping never holds them pending inside the tile loop.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  refill(0);

  int st_cur = 0;  // stage of the tile being computed
  for (;;) {
    // ---- one item ---------------------------------------------------------
    float m_run = -INFINITY;  // running max of scale*log2(e)*s (possibly stale by < slack)
    float l_run = 0.f;        // lane-partial running sum
    f32x16 acc[C::NDT];
#pragma unroll
    for (int u = 0; u < C::NDT; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[u][i] = 0.f;

    for (int u = 0; u < cur_cnt; ++u) {
      // Column of the tile to prefetch this step (scalar load, consumed after
      // the barrier).  The tiles issued after the current one are the only
      // loads allowed in flight; the barrier then makes every wave's part of
      // the current tile visible and frees the stage computed one step ago.
      // (The column load is unconditional, from a valid dummy entry past the
      // stream, so that the wave waits for it only at the barrier.)
      bool in_next;
      const int src = inflight < C::NSTAGE ? stream_src(u + inflight, in_next) : -1;
      const int jn = ld_uniform(col_src, src >= 0 ? src : 0);
      if (inflight > 1)
        wait_vm(C::DPW);
      else
        wait_vm(0);
      __syncthreads();
      if (src >= 0) issue(jn, in_next);
      const uint32_t ks = lds0 + uint32_t(st_cur) * C::STAGEB;
      const uint32_t vs = ks + C::TILEB;
      const int valid = static_cast<int>(vq & 0xffu);

      // S^T tile: lane (ql, hh) holds keys key0 + 8(i/4) + 4hh + (i%4) of query ql.
      // A subtile's K operands are all read before its MFMAs (one LDS round
      // trip, not one per MFMA).
      const f32x16 zero = {};
      f32x16 s[C::NKT];
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt) {
        const int key = (kh * C::NKT + kt) * 32 + ql;
        bf16x8 ka[C::NDC];
#pragma unroll
        for (int c = 0; c < C::NDC; ++c) ka[c] = lds_read16(ks + swz<C::ROWB>(key, 2 * c + hh));
#pragma unroll
        for (int c = 0; c < C::NDC; ++c)
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qf[c], c == 0 ? zero : s[kt], 0,
                                                          0, 0);
      }

      // V^T operands of O^T += V^T P^T.  For the 16-key step kb, V^T rows
      // d = 32u + (lane % 32) need keys kb + 4hh + e and kb + 8 + 4hh + e
      // (e = 0..3): lane t of each 16-lane block points at key row t / 4 and
      // columns 4 (t % 4) .. +3 of its block's 16 d values, and the transposing
      // read returns to every lane the four keys of its own d column.  When
      // they fit in the registers the K operands held, all are read here and
      // land while the softmax runs; otherwise one key subtile's at a time.
      constexpr bool kEarlyV = C::NKT * C::NDT <= 4;
      const int tr_row = 4 * hh + ((lane & 15) >> 2);
      const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      v4s vlo[C::NKT][2][C::NDT], vhi[C::NKT][2][C::NDT];
      auto read_v = [&](int kt) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const int kb = (kh * C::NKT + kt) * 32 + 16 * c2;
#pragma unroll
          for (int u2 = 0; u2 < C::NDT; ++u2) {
            const int col = 32 * u2 + tr_col;
            vlo[kt][c2][u2] = lds_read_tr(vs + swz<C::ROWB>(kb + tr_row, col >> 3) + (col & 7) * 2);
            vhi[kt][c2][u2] =
                lds_read_tr(vs + swz<C::ROWB>(kb + 8 + tr_row, col >> 3) + (col & 7) * 2);
          }
        }
      };
      if (kEarlyV) {
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt) read_v(kt);
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
      // Probabilities against the running max as it stands.  Past a row's
      // first tile the tile's max is needed only when a probability could
      // leave the safe range, which some lane's partial row sum shows (above
      // kSumCap, or not finite), or while a row has no max yet; then each
      // row's max is raised to the tile's, its state rescaled and the tile's
      // probabilities recomputed.  The first tile takes its max up front.
      // Row sums in four independent chains (no long serial add dependency).
      float lt;
      bf16x8 pb[C::NKT][2];
      auto probs = [&]() {
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        float ls[4];
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
        lt = (ls[0] + ls[1]) + (ls[2] + ls[3]);
      };
      auto raise_max = [&]() {
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
        mx = fmaxf(mx, other_half(mx));
        const float mt = mx * sl2;
        const bool up = mt > m_run;
        // A row's first finite max is adopted without touching its (zero) state.
        const float alpha = (up && m_run != -INFINITY) ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int u2 = 0; u2 < C::NDT; ++u2)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[u2][i] *= alpha;
        m_run = up ? mt : m_run;
      };
      if (u == 0) raise_max();
      probs();
      if (u != 0 &&
          __builtin_expect(
              __builtin_amdgcn_ballot_w64(!(lt <= kSumCap) || m_run == -INFINITY) != 0, 0)) {
        raise_max();
        probs();
      }
      l_run += lt;

      // O^T += V^T P^T.
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt) {
        if (!kEarlyV) read_v(kt);
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int u2 = 0; u2 < C::NDT; ++u2) {
            const bf16x8 a = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(vlo[kt][c2][u2], vhi[kt][c2][u2], 0, 1, 2, 3, 4,
                                                5, 6, 7));
            acc[u2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kt][c2], acc[u2], 0, 0, 0);
          }
      }

      // Retire the tile.
      st_cur = st_cur + 1 == C::NSTAGE ? 0 : st_cur + 1;
      vq >>= 8;
      --inflight;
    }

    // ---- epilogue: merge the key halves through the stage before st_cur ---
    // (the last computed tile's stage; no load targets it until the next
    // barrier of the tile loop).
    const int st_free = st_cur == 0 ? C::NSTAGE - 1 : st_cur - 1;
    float l_half = l_run + other_half(l_run);
    __syncthreads();  // every wave is done with that stage and the merge area
    float* mg = reinterpret_cast<float*>(smem + size_t(st_free) * C::STAGEB) +
                size_t(qg) * 64 * C::NDT * 16;
    if (kh == 1) {
#pragma unroll
      for (int u = 0; u < C::NDT; ++u)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4*>(mg + ((u * 4 + g) * 64 + lane) * 4) =
              f32x4{acc[u][4 * g], acc[u][4 * g + 1], acc[u][4 * g + 2], acc[u][4 * g + 3]};
      ml[(qg * 2) * 64 + lane] = m_run;
      ml[(qg * 2 + 1) * 64 + lane] = l_half;
    }
    // The item after next: the claim made one item ago (work list) or the
    // next static round; wave 0 publishes it after the merge area.
    int* xk = reinterpret_cast<int*>(ml + C::ML_FLOATS);
    if (queue && wave == 0) {
      const int t = claim_out ? __builtin_amdgcn_readfirstlane(ticket) : -1;
      if (lane == 0) {
        *xk = src.claimed(t);
        if (claim_out) src.retire(ctr, t);
      }
    }
    __syncthreads();
    const int k_nn = queue ? *xk : src.stat(round);
    if (kh == 0) {
      const float m1 = ml[(qg * 2) * 64 + lane];
      const float l1 = ml[(qg * 2 + 1) * 64 + lane];
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
      const int bh = cur_row / nb;
      const int q = qg * 32 + ql;
      const int qrow = (cur_row - bh * nb) * BLK + q;
      if (cur_slot >= 0) {
        // Partial result of one chunk: unnormalised acc, running max (log2
        // units) and running sum, combined with the row's other chunks by
        // merge_kernel.
        float* po = part + size_t(cur_slot) * BLK * (HD + 2);
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
      } else if (qrow < N) {
        const size_t head = size_t(bh) * size_t(N) * HD;
        const float inv = l_half > 0.f ? 1.f / l_half : 0.f;
        uint16_t* orow = O + head + size_t(qrow) * HD;
        // With a residual, O = attention + R, summed in fp32, rounded once.
        const uint16_t* rrow = RES ? R + head + size_t(qrow) * HD : nullptr;
#pragma unroll
        for (int u = 0; u < C::NDT; ++u)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d0 = 32 * u + 8 * g + 4 * hh;
            f32x4 y = f32x4{acc[u][4 * g + 0], acc[u][4 * g + 1], acc[u][4 * g + 2],
                            acc[u][4 * g + 3]} * inv;
            if (RES) {
              const uint2 rv = *reinterpret_cast<const uint2*>(rrow + d0);
              y += f32x4{bf16_lo(rv.x), bf16_hi(rv.x), bf16_lo(rv.y), bf16_hi(rv.y)};
            }
            *reinterpret_cast<uint2*>(orow + d0) =
                make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
          }
        if (hh == 0 && LSE != nullptr) {
          LSE[size_t(bh) * N + qrow] =
              l_half > 0.f ? (m_run + __builtin_amdgcn_logf(l_half)) * 0.69314718055994531f
                           : -INFINITY;
        }
      }
    }

    // ---- advance to the next item ----------------------------------------
    k_cur = k_nxt;
    k_nxt = k_nn;
    ++round;
    if (k_cur < 0) break;
    cur_row = nxt_row;
    cur_c0 = nxt_c0;
    cur_cnt = nxt_cnt;
    cur_slot = nxt_slot;
    desc_cur = desc_nxt;
#pragma unroll
    for (int c = 0; c < C::NDC; ++c) qf[c] = qn[c];
    // The copy above waited for the query loads; make that explicit so they
    // are never seen as pending inside the tile loop.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    load_item(k_nxt, nxt_row, nxt_c0, nxt_cnt, nxt_slot);
    claim_out = queue && k_nxt >= 0;
    if (claim_out && wave == 0 && lane == 0) ticket = src.claim(ctr);
    desc_nxt = kv_desc(nxt_row);
    load_q(nxt_row, qn);
    refill(0);
  }
  wait_vm(0);  // no load may still target LDS when the workgroup retires
}

// ---------------------------------------------------------------------------
// Wide wavefronts for 64-row blocks at head dim 64 or 128.
//
// Two wavefronts per workgroup.  Wave h owns keys 32h .. 32h+31 of every
// 64-key tile for all 64 query rows of the block (two 32-row query groups),
// so every K or V^T operand it reads from LDS feeds two MFMAs: half the LDS
// traffic, DMA issue and scalar work per FLOP of 32-row wavefronts.  The waves
// share no tile data: each streams its own halves of K and V into its own
// two-stage LDS ring (one tile ahead) and waits only on its own loads, so the
// tile loop has no barrier.  The next item's query tile is staged in LDS while
// the current item runs; the two key halves meet once per item, in the
// epilogue, through the stages the last tile freed.
//
// At head dim 128 everything doubles along d (40 -> 80 KB of LDS: two workgroups
// per CU, one wavefront per SIMD, which may then use the whole register file).
template <int HD_>
struct Wide {
  static constexpr int BLK = 64, HD = HD_, ROWB = 2 * HD;
  static constexpr int NT = 128;                     // two wavefronts
  static constexpr int NDC = HD / 16;                // k-steps of the QK^T product
  static constexpr int NDT = HD / 32;                // 32-wide d subtiles of the output
  static constexpr int HALFB = 32 * ROWB;            // one wave's half of a K or V tile
  static constexpr int LPH = HALFB / 1024;           // 16-byte-per-lane loads per half tile
  static constexpr int STAGEB = 2 * HALFB;           // K half, then V half
  static constexpr int RINGB = 2 * STAGEB;           // two stages per wave
  static constexpr int QB = BLK * ROWB;              // staged query tile
  static constexpr size_t LDS_BYTES = 2 * RINGB + QB;  // 40 KB (80 KB at head dim 128)
  static_assert(NDT * 16 * 4 * 64 == STAGEB, "one query group's accumulator fills a stage");
  static_assert(HD == 64 || HD == 128, "head dim 64 or 128");
};

template <int HD_, bool RES>
__global__ __launch_bounds__(Wide<HD_>::NT) __attribute__((amdgpu_waves_per_eu(HD_ == 64 ? 2 : 1))) void fwd_wide_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, const int32_t* __restrict__ work, int32_t n_items,
    int32_t n_merges, int32_t N, int32_t nb, int32_t n_rows, float sl2, uint16_t* __restrict__ O,
    float* __restrict__ LSE, float* __restrict__ part, int32_t* __restrict__ ctr, int32_t n_slots,
    int32_t* __restrict__ mctr, const uint16_t* __restrict__ R) {
  using W = Wide<HD_>;
  constexpr int BLK = W::BLK, HD = W::HD, NDC = W::NDC, NDT = W::NDT;
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((BSA_LDS uint8_t*)smem));

  const int lane = threadIdx.x & 63;
  const int kh = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // key half of this wave
  const int ql = lane & 31;  // query column (within a group) / key row of the MFMA tiles
  const int hh = lane >> 5;  // which half of the k / row dimension the lane feeds
  const uint32_t head_bytes = static_cast<uint32_t>(size_t(N) * W::ROWB);
  const int nnz = ld_uniform(row_ptr, n_rows);
  const uint32_t ring = lds0 + uint32_t(kh) * W::RINGB;
  const uint32_t qarea = lds0 + 2u * W::RINGB;
  // head(row) = row / nb.  For nb >= 2, with magic = floor(2^32 / nb) + 1 the
  // multiply-high estimate is never low and, for row < 2^31, at most one too
  // high; one correction makes it exact.  (nb = 1 would need magic = 2^32 + 1.)
  const uint32_t nb_magic =
      nb > 1 ? static_cast<uint32_t>((uint64_t(1) << 32) / uint32_t(nb)) + 1u : 0u;
  auto head_of = [&](int row) -> int {
    if (nb == 1) return row;
    int h = static_cast<int>(__umulhi(static_cast<uint32_t>(row), nb_magic));
    if (row - h * nb < 0) --h;
    return h;
  };

  auto load_item = [&](int k, int& row, int& c0, int& cnt, int& slot) {
    row = -1;
    c0 = cnt = 0;
    slot = -1;
    if (k < 0 || k >= n_items) return;
    int r, b, e, sl;
    if (work) {
      r = ld_uniform(work, 4 * size_t(k));
      b = ld_uniform(work, 4 * size_t(k) + 1);
      e = ld_uniform(work, 4 * size_t(k) + 2);
      sl = ld_uniform(work, 4 * size_t(k) + 3);
    } else {
      r = k;
      b = ld_uniform(row_ptr, k);
      e = ld_uniform(row_ptr, k + 1);
      sl = -1;
    }
    if (r < 0 || r >= n_rows) return;
    b = min(max(b, 0), nnz);
    e = min(max(e, b), nnz);
    row = r;
    c0 = b;
    cnt = e - b;
    slot = sl;
  };

  // Source offsets of the chunks that land at this lane's swizzled LDS
  // positions in segments 0 and 1 (relative to their segment); at head dim 128
  // (4 rows per segment, a swizzle of period 16 rows) in segments 0 .. 3.
  uint32_t ve = 0, vo = 0, vs[4] = {0, 0, 0, 0};
  if constexpr (HD == 64) {
    const int r0 = lane >> 3, p = lane & 7;
    ve = uint32_t(r0) * W::ROWB + uint32_t((p ^ chunk_swizzle<W::ROWB>(r0)) << 4);
    vo = uint32_t(r0) * W::ROWB + uint32_t((p ^ chunk_swizzle<W::ROWB>(8 + r0)) << 4);
  } else {
    const int r0 = lane >> 4, p = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vs[i] = uint32_t(r0) * W::ROWB + uint32_t((p ^ chunk_swizzle<W::ROWB>(4 * i + r0)) << 4);
  }
  // One 32-row half tile (source offset tb) into LDS at dst: W::LPH loads.
  auto dma_rows = [&](v4i desc, uint32_t tb, uint32_t dst) {
    if constexpr (HD == 64) {
      dma_half(desc, ve + tb, vo + tb, dst);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        dma16x4(desc, vs[0] + tb + 4096u * h, vs[1] + tb + 4096u * h, vs[2] + tb + 4096u * h,
                vs[3] + tb + 4096u * h, dst + 4096u * h);
    }
  };

  // Buffer descriptor over head bh of tensor T (an empty range when row < 0).
  auto head_desc = [&](const uint16_t* T, int row, int bh) -> v4i {
    v4i d = make_desc(T + size_t(bh) * size_t(N) * HD, row >= 0 ? head_bytes : 0u);
#pragma unroll
    for (int w = 0; w < 4; ++w) d[w] = __builtin_amdgcn_readfirstlane(d[w]);
    return d;
  };

  // Count of this wave's vector-memory operations (loads into LDS, stores,
  // claims) in issue order.  Operations retire in order, so an operation
  // issued when the count read `stamp` is complete once seq - stamp younger
  // ones remain outstanding.  Operations left out of the count only make a
  // wait stricter.
  int seq = 0;
  // This wave's half of the query tile of CSR row `row` into the staging area.
  int q_stamp = 0;
  auto stage_q = [&](int row, int bh) {
    if (row < 0) return;
    const int qb = row - bh * nb;
    const uint32_t tb = uint32_t(qb) * (BLK * W::ROWB) + uint32_t(kh) * W::HALFB;
    dma_rows(head_desc(Q, row, bh), tb, qarea + uint32_t(kh) * W::HALFB);
    seq += W::LPH;
    q_stamp = seq;
  };
  // Query fragments (B operand of S^T = K Q^T) from the staging area: lane
  // holds d = 16c + 8hh .. +7 of query row 32g + ql.
  auto read_q = [&](bf16x8 (&qf)[2][NDC]) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int c = 0; c < NDC; ++c) qf[g][c] = lds_read16(qarea + swz<W::ROWB>(32 * g + ql, 2 * c + hh));
  };

  // ---- item source --------------------------------------------------------
  ItemSource src;
  src.init(work, n_items, n_merges, n_rows);
  const bool queue = work != nullptr;
  int k_cur = src.stat(0), k_nxt = src.stat(1);
  int round = 2;           // static round of the item after next (no work list)
  bool claim_out = false;  // a claim for the item after next is in flight
  int ticket = -1;         // its claim number, in lane 0 of wave 0
  if (k_cur < 0) return;
  claim_out = queue && k_nxt >= 0;
  if (claim_out && kh == 0 && lane == 0) ticket = src.claim(ctr);

  // The claimed item after next, resolved by wave 0 one step before the
  // current item ends and published to wave 1 in the epilogue.
  bool nn_known = false;
  int nn_k = -1, nn_row = -1, nn_c0 = 0, nn_cnt = 0, nn_slot = -1;

  // ---- stream state -------------------------------------------------------
  int cur_row, cur_c0, cur_cnt, cur_slot, nxt_row, nxt_c0, nxt_cnt, nxt_slot;
  load_item(k_cur, cur_row, cur_c0, cur_cnt, cur_slot);
  load_item(k_nxt, nxt_row, nxt_c0, nxt_cnt, nxt_slot);
  int cur_bh = cur_row >= 0 ? head_of(cur_row) : 0;
  int nxt_bh = nxt_row >= 0 ? head_of(nxt_row) : 0;
  v4i kd_cur = head_desc(K, cur_row, cur_bh), vd_cur = head_desc(V, cur_row, cur_bh);
  v4i kd_nxt = head_desc(K, nxt_row, nxt_bh), vd_nxt = head_desc(V, nxt_row, nxt_bh);
  // Wave 0: read the claim for the item after next and start loading its
  // record.  Called where the only load in flight is the tile about to be
  // used, so the wait for the claim costs nothing extra.
  auto resolve_claim = [&]() {
    const int t = __builtin_amdgcn_readfirstlane(ticket);
    nn_k = src.claimed(t);
    if (lane == 0) src.retire(ctr, t);
    nn_known = true;
    load_item(nn_k, nn_row, nn_c0, nn_cnt, nn_slot);
  };


  // K and V stream as half tiles through the wave's two-stage ring, K one tile
  // further ahead than V, so that the scores of tile u + 1 are formed while the
  // softmax of tile u runs and the matrix cores and the vector ALU of the
  // wavefront overlap.  Position p of the current item (p = cur_cnt: the next
  // item's first tile) uses stage (ib + p) & 1 of both the K and the V half of
  // the ring.  k_last and v_last are the issue stamps of the latest K and V
  // loads.
  int ib = 0, k_last = 0, v_last = 0;
  auto valid_of = [&](int j) -> int { return (j >= 0 && j < nb) ? min(BLK, N - j * BLK) : 0; };
  auto issue = [&](v4i d, int j, int p, bool is_v) {
    const bool ok = j >= 0 && j < nb;
    const uint32_t tb = ok ? uint32_t(j) * (BLK * W::ROWB) + uint32_t(kh) * W::HALFB : head_bytes;
    dma_rows(d, tb, ring + uint32_t((ib + p) & 1) * W::STAGEB + (is_v ? uint32_t(W::HALFB) : 0u));
    seq += W::LPH;
    if (is_v)
      v_last = seq;
    else
      k_last = seq;
  };
  // Column of the next item's first tile, or -1.
  auto first_of_next = [&]() -> int { return nxt_cnt > 0 ? ld_uniform(col_idx, nxt_c0) : -1; };

  // Start-up: the first query tile and the first item's first K and V tiles.
  bf16x8 qf[2][NDC];
  stage_q(cur_row, cur_bh);
  if (cur_cnt > 0) {
    const int j0 = ld_uniform(col_idx, cur_c0);
    issue(kd_cur, j0, 0, false);
    issue(vd_cur, j0, 0, true);
  }
  wait_vm_n(seq - q_stamp);
  lds_barrier();
  read_q(qf);
  lds_barrier();
  stage_q(nxt_row, nxt_bh);

  // Chunk partials and their merge.  A wave's partial stores (agent-scope
  // coherent) are known complete one epilogue later, where that epilogue's
  // first wait covers them (after the last item: at once, by a full wait).
  // The wave then counts its query group of that chunk in; the wave whose
  // count-in completes the number of chunks combines the group's partials of
  // every chunk of the row and clears the count.  The count-in's result is
  // read on every path before the epilogue's stores, so that no memory result
  // is left in flight into the loop (the compiler's wait bookkeeping would
  // then drain the tile prefetch there).
  int rel_slot = -1;  // chunk whose partial this wave stored, not yet counted in
  int st_stamp = 0;   // issue stamp after the latest epilogue's stores
  const int32_t* slot_merge =
      work ? work + 4 * size_t(n_items) + 3 * size_t(n_merges) + 2 + src.ng : nullptr;
  const int32_t* merges = work ? work + 4 * size_t(n_items) : nullptr;
  // (Merge indices pass through readfirstlane: they are wave-uniform, and the
  // compiler must keep them, and the loads they address, scalar.)
  auto merge_of = [&](int slot) -> int {
    const int m = (slot >= 0 && slot < n_slots) ? ld_uniform(slot_merge, slot) : -1;
    return __builtin_amdgcn_readfirstlane((m >= 0 && m < n_merges && m < n_slots) ? m : -1);
  };
  // Count this wave's query group of merge m in; lane 0 gets the count before.
  auto count_in = [&](int m) -> int {
    int old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(mctr + 2 * m + kh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return old;
  };
  // Whether a count-in (old count in lane 0) completed merge m (m >= 0).
  auto completes = [&](int m, int old) -> bool {
    return old == ld_uniform(merges, 3 * size_t(m) + 2) - 1;
  };
  // Combine query group kh of cut row `merges[m]` from its chunks' partials:
  // with M = max_c m_c, O = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c and
  // LSE = (M + log2 L) ln 2.  Lane (ql, hh) owns query 32 kh + ql, columns
  // 32 hh .. +31.  Returns the number of stores issued.
  //
  // Ordering: a chunk's partial stores use the device-coherent cache policy
  // and complete (vmcnt) before its relaxed count-in, which is the release
  // side; the wave whose count-in completes the row acquires (agent scope)
  // before it reads the other chunks' partials.
  auto merge_group = [&](int m) -> int {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (lane == 0)
      __hip_atomic_store(mctr + 2 * m + kh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int r = ld_uniform(merges, 3 * size_t(m));
    const int slot0 = ld_uniform(merges, 3 * size_t(m) + 1);
    const int nch = ld_uniform(merges, 3 * size_t(m) + 2);
    if (r < 0 || r >= n_rows || nch < 1 || slot0 < 0 || slot0 >= n_slots) return 0;
    constexpr uint32_t kSlotFloats = BLK * (HD + 2);
    const int nc = min(nch, n_slots - slot0);
    const __amdgpu_buffer_rsrc_t pr =
        make_rsrc(part + size_t(slot0) * kSlotFloats, uint32_t(nc) * kSlotFloats * 4u);
    const int q = 32 * kh + ql;
    constexpr int NJ = HD / 8;  // 16-byte pieces of the lane's HD / 2 fp32 columns
    const uint32_t qoff = uint32_t(q * HD + (HD / 2) * hh) * 4u;
    float M = -INFINITY, L = 0.f;
    f32x4 o[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Chunks are read kMB at a time (their loads in flight together); the
    // batch is kept small so that the merge does not set the kernel's
    // register budget.
    constexpr int kMB = 2;
    for (int c0 = 0; c0 < nc; c0 += kMB) {
      f32x4 a[kMB][NJ];
      float mc[kMB], lc[kMB];
#pragma unroll
      for (int t = 0; t < kMB; ++t) {
        // Chunks past the row's last read past the range: zeros, weight 0.
        const uint32_t cb = uint32_t(c0 + t) * kSlotFloats * 4u;
        mc[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            pr, cb + uint32_t(BLK * HD + q) * 4u, 0, kAgentScope));
        lc[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            pr, cb + uint32_t(BLK * HD + BLK + q) * 4u, 0, kAgentScope));
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          a[t][j] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, cb + qoff + 16u * j, 0, kAgentScope));
      }
#pragma unroll
      for (int t = 0; t < kMB; ++t) {
        if (c0 + t >= nc) break;
        const float mn = fmaxf(M, mc[t]);
        const float wo = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - mn);
        const float wc = mc[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc[t] - mn);
        L = L * wo + lc[t] * wc;
#pragma unroll
        for (int j = 0; j < NJ; ++j) o[j] = o[j] * wo + a[t][j] * wc;
        M = mn;
      }
    }
    const int bh = head_of(r);
    const int qrow = (r - bh * nb) * BLK + q;
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const __amdgpu_buffer_rsrc_t orsc = make_rsrc(O + size_t(bh) * size_t(N) * HD, head_bytes);
    const uint32_t ob = uint32_t(qrow) * W::ROWB + uint32_t((HD / 2) * hh) * 2u;
    // O = attention (+ R, summed in fp32), rounded once to bf16.
    v4u rr[NJ / 2];
    if (RES) {
      const __amdgpu_buffer_rsrc_t rrsc = make_rsrc(R + size_t(bh) * size_t(N) * HD, head_bytes);
#pragma unroll
      for (int j = 0; j < NJ / 2; ++j) rr[j] = __builtin_amdgcn_raw_buffer_load_b128(rrsc, ob + 16u * j, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NJ / 2; ++j) {
      f32x4 x = o[2 * j] * inv, y = o[2 * j + 1] * inv;
      if (RES) {
        x += f32x4{bf16_lo(rr[j][0]), bf16_hi(rr[j][0]), bf16_lo(rr[j][1]), bf16_hi(rr[j][1])};
        y += f32x4{bf16_lo(rr[j][2]), bf16_hi(rr[j][2]), bf16_lo(rr[j][3]), bf16_hi(rr[j][3])};
      }
      const v4u w = v4u{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(y[0], y[1]),
                        pack_bf16x2(y[2], y[3])};
      __builtin_amdgcn_raw_buffer_store_b128(w, orsc, ob + 16u * j, 0, 0);
    }
    if (LSE == nullptr) return NJ / 2;
    const __amdgpu_buffer_rsrc_t lrsc =
        make_rsrc(LSE + size_t(bh) * size_t(N), static_cast<uint32_t>(N) * 4u);
    const float lv = L > 0.f ? (M + __builtin_amdgcn_logf(L)) * 0.69314718055994531f : -INFINITY;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lv), lrsc,
                                          hh == 0 ? uint32_t(qrow) * 4u : uint32_t(N) * 4u, 0, 0);
    return NJ / 2 + 1;
  };

  // Lane position of the transposing V^T reads: for the 16-key step c2, V^T
  // rows d = 32u + (lane % 32) need keys 16c2 + 4hh + e and 16c2 + 8 + 4hh + e
  // (e = 0..3): lane t of each 16-lane block points at key row t / 4 and
  // columns 4 (t % 4) .. +3 of its block's 16 d values, and the transposing
  // read returns to every lane the four keys of its own d.  V^T rows 16..31 of
  // a tile (the second 16-key step) sit 2048 bytes past rows 0..15 and
  // swizzle alike.
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  uint32_t koff[NDC], voff[2 * NDT];  // lane offsets of the K and V^T reads within a stage
#pragma unroll
  for (int c = 0; c < NDC; ++c) koff[c] = swz<W::ROWB>(ql, 2 * c + hh);
#pragma unroll
  for (int u2 = 0; u2 < NDT; ++u2)
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) {
      const int col = 32 * u2 + tr_col;
      voff[2 * u2 + hl] = W::HALFB + swz<W::ROWB>(8 * hl + tr_row, col >> 3) + (col & 7) * 2;
    }
  auto stage_at = [&](int p) -> uint32_t { return ring + uint32_t((ib + p) & 1) * W::STAGEB; };
  auto read_k = [&](uint32_t st, bf16x8 (&ka)[NDC]) {
#pragma unroll
    for (int c = 0; c < NDC; ++c) ka[c] = lds_read16(st + koff[c]);
  };
  auto read_v = [&](uint32_t st, v4s (&vlo)[2][NDT], v4s (&vhi)[2][NDT]) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int u2 = 0; u2 < NDT; ++u2) {
        vlo[c2][u2] = lds_read_tr(st + voff[2 * u2] + uint32_t(16 * W::ROWB) * c2);
        vhi[c2][u2] = lds_read_tr(st + voff[2 * u2 + 1] + uint32_t(16 * W::ROWB) * c2);
      }
  };
  // S^T of query group g: lane (ql, hh) holds keys 8(i/4) + 4hh + (i%4) (of
  // this half) of query 32g + ql.
  auto scores_g = [&](int g, const bf16x8 (&ka)[NDC], f32x16& s) {
    const f32x16 zero = {};
#pragma unroll
    for (int c = 0; c < NDC; ++c)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qf[g][c], c == 0 ? zero : s, 0, 0, 0);
  };
  // Keys at or past the tile's valid count score -inf (both groups).  Lane
  // element i is key 32kh + 4hh + o_i of the tile, o_i = 8(i/4) + (i%4); bit o
  // of `bad` marks offsets at or past the valid count, and min(s, +-inf) keeps
  // or drops the score without per-element compare masks.
  auto mask = [&](f32x16 (&s)[2], int valid) {
    const int lim = valid - (32 * kh + 4 * hh);
    const uint32_t bad = lim <= 0 ? 0xffffffffu : (lim >= 32 ? 0u : (0xffffffffu << lim));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int o = 8 * (i >> 2) + (i & 3);
      const float cap = __uint_as_float(0x7f800000u | (((bad >> o) & 1u) << 31));
      s[0][i] = __builtin_fminf(s[0][i], cap);
      s[1][i] = __builtin_fminf(s[1][i], cap);
    }
  };
  // Row maxima of a score tile in log2 units (both key halves of the wave).
  auto tile_max = [&](const f32x16 (&s)[2], float (&mt)[2]) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float mx = vmax(s[g][0], s[g][1]);
#pragma unroll
      for (int i = 2; i < 16; ++i) mx = vmax(mx, s[g][i]);
      // The other half-wave holds the other 16 keys of the same queries.
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mt[g] = vmax(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sl2;
    }
  };

  for (;;) {
    // ---- one item ---------------------------------------------------------
    float m_run[2] = {kNoMax, kNoMax};  // running max of scale*log2(e)*s
    float l_run[2] = {0.f, 0.f};        // lane-partial running sums
    f32x16 acc[2][NDT];                 // [query group][32-wide d subtile]
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int u = 0; u < NDT; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][u][i] = 0.f;

    // Lazy rescale: only when some row's max grew by more than the slack; a
    // row's first finite max is adopted without touching its zero state.
    auto adopt_max = [&](const float (&mt)[2]) {
      bool need[2], rescale[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        need[g] = mt[g] > m_run[g] + kRescaleSlack;
        rescale[g] = need[g] && m_run[g] != kNoMax;
      }
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(rescale[0] || rescale[1]) != 0, 0)) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const float alpha = rescale[g] ? __builtin_amdgcn_exp2f(m_run[g] - mt[g]) : 1.f;
          l_run[g] *= alpha;
#pragma unroll
          for (int u2 = 0; u2 < NDT; ++u2)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[g][u2][i] *= alpha;
        }
      }
#pragma unroll
      for (int g = 0; g < 2; ++g) m_run[g] = need[g] ? mt[g] : m_run[g];
    };
    // Softmax numerators of query group g: P in bf16 only as the MFMA operand;
    // the row sum adds the fp32 values in four independent chains.
    auto probs_g = [&](int g, const f32x16& s, bf16x8 (&pb)[2]) {
      float ls[4];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[i], sl2, -m_run[g]));
        if (i < 4)
          ls[i] = p;
        else
          ls[i & 3] += p;
        pb[i >> 3][i & 7] = static_cast<__bf16>(p);
      }
      l_run[g] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    };
    // Query group g: the softmax numerators of tile u (scores sc) interleaved
    // with the four MFMAs of tile u + 1's scores (into sn), a quarter of the
    // vector work after each, so that both run at once.
    auto phase = [&](int g, const bf16x8 (&ka)[NDC], const f32x16& sc, f32x16& sn, bf16x8 (&pb)[2]) {
      constexpr int EPC = 16 / NDC;  // softmax elements per score MFMA
      const f32x16 zero = {};
      float p[16];
      float ls[4];
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qf[g][c], c == 0 ? zero : sn, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const int i = EPC * c + e;
          p[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], sl2, -m_run[g]));
          if (i < 4)
            ls[i & 3] = p[i];
          else
            ls[i & 3] += p[i];
        }
        if ((EPC * (c + 1)) % 8 == 0) {
          const int h8 = EPC * (c + 1) / 8 - 1;
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[h8][e] = static_cast<__bf16>(p[8 * h8 + e]);
        }
        if constexpr (HD == 64) {  // (at head dim 128 the compiler's order measured as fast)
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // the MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 14, 0);  // its share of the softmax
        }
      }
      l_run[g] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    };
    // O^T += V^T P^T, one V^T operand per 16-key step and d half, shared by both
    // query groups.
    auto pv = [&](const v4s (&vlo)[2][NDT], const v4s (&vhi)[2][NDT], const bf16x8 (&pb)[2][2]) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int u2 = 0; u2 < NDT; ++u2) {
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(vlo[c2][u2], vhi[c2][u2], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int g = 0; g < 2; ++g)
            acc[g][u2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[g][c2], acc[g][u2], 0, 0, 0);
        }
    };

    const int cnt = cur_cnt;
    const int j0n = first_of_next();
    // Columns of positions u + 1 (its V is issued in step u and its scores
    // formed there) and u + 2 (its K is issued in step u), looked up one step
    // early.
    int jv = cnt > 1 ? ld_uniform(col_idx, cur_c0 + 1) : 0;
    int jk = cnt > 2 ? ld_uniform(col_idx, cur_c0 + 2) : j0n;
    // Row maxima of the tile whose scores are held (mt) are adopted at the
    // start of the step that runs its softmax; a tile with keys past N
    // (valid count vs < BLK, only the last block of a head) has its scores
    // masked and its maxima recomputed first.  Before the step's own loads,
    // the latest are V(u) and K(u + 1).
    float mt[2];
    int vs = BLK;  // valid keys of the tile whose scores are held
    auto settle = [&](f32x16 (&sc)[2]) {
      if (__builtin_expect(vs < BLK, 0)) {
        mask(sc, vs);
        tile_max(sc, mt);
      }
      adopt_max(mt);
    };
    // One pipelined step: softmax and P V of tile u (scores in sc), scores and
    // unmasked maxima of tile u + 1 (< cnt) into sn.  Three phases, each
    // pairing matrix work with independent vector work: (A) group 0's softmax
    // with group 0's next scores, (B) the same for group 1, (C) P V with the
    // next row maxima.
    auto step = [&](int u, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
      // Wave 0 reads the claim for the item after next where the only loads
      // in flight are the ones this step waits for anyway.
      if (queue && kh == 0 && claim_out && !nn_known && u + 2 == cnt) resolve_claim();
      settle(sc);
      issue(vd_cur, jv, u + 1, true);
      int issued = W::LPH;
      if (u + 2 < cnt) {
        issue(kd_cur, jk, u + 2, false);
        issued = 2 * W::LPH;
      } else if (jk >= 0) {  // the next item's first tile
        issue(kd_nxt, jk, u + 2, false);
        issued = 2 * W::LPH;
      }
      vs = valid_of(jv);
      jv = jk;
      jk = u + 3 < cnt ? ld_uniform(col_idx, cur_c0 + u + 3) : j0n;
      wait_vm_n(issued);
      bf16x8 ka[NDC];
      v4s vlo[2][NDT], vhi[2][NDT];
      bf16x8 pb[2][2];
      read_k(stage_at(u + 1), ka);
      read_v(stage_at(u), vlo, vhi);
      __builtin_amdgcn_sched_barrier(0);
      phase(0, ka, sc[0], sn[0], pb[0]);
      __builtin_amdgcn_sched_barrier(0);
      phase(1, ka, sc[1], sn[1], pb[1]);
      __builtin_amdgcn_sched_barrier(0);
      pv(vlo, vhi, pb);
      tile_max(sn, mt);
      if constexpr (HD == 64) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one P V MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // row max of the next tile
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // Item start: K(0) and V(0) were issued with the previous item (or at
    // start-up).  Issue K(1), which is the next item's first tile when this
    // item has one tile; an item without tiles issues the next item's first
    // K and V.
    const int k0_stamp = k_last;
    if (cnt > 1)
      issue(kd_cur, jv, 1, false);
    else if (j0n >= 0) {
      issue(kd_nxt, j0n, cnt, false);
      if (cnt == 0) issue(vd_nxt, j0n, 0, true);
    }
    if (cnt > 0) {
      f32x16 sa[2], sb[2];
      // Prologue: the scores of the first tile and their maxima.
      {
        vs = valid_of(ld_uniform(col_idx, cur_c0));
        wait_vm_n(seq - k0_stamp);
        bf16x8 ka[NDC];
        read_k(stage_at(0), ka);
        scores_g(0, ka, sa[0]);
        scores_g(1, ka, sa[1]);
        tile_max(sa, mt);
      }
      // Pipelined steps u = 0 .. cnt - 2, two per trip so that the score tiles
      // alternate between sa and sb without copies.
      int u = 0;
      while (u + 2 < cnt) {
        step(u, sa, sb);
        step(u + 1, sb, sa);
        u += 2;
      }
      if (u + 1 < cnt) {
        step(u, sa, sb);
        ++u;
#pragma unroll
        for (int g = 0; g < 2; ++g) sa[g] = sb[g];
      }
      // The last tile: its softmax and P V; the next item's first V follows
      // its first K.
      settle(sa);
      if (queue && kh == 0 && claim_out && !nn_known) resolve_claim();
      const int v_stamp = v_last;
      if (j0n >= 0) issue(vd_nxt, j0n, cnt, true);
      wait_vm_n(seq - v_stamp);
      v4s vlo[2][NDT], vhi[2][NDT];
      bf16x8 pb[2][2];
      read_v(stage_at(cnt - 1), vlo, vhi);
      probs_g(0, sa[0], pb[0]);
      probs_g(1, sa[1], pb[1]);
      pv(vlo, vhi, pb);
    }

    // ---- epilogue -----------------------------------------------------------
    // The next item's query tile (this wave's half) and the previous
    // epilogue's partial stores, if any, are complete.
    wait_vm_n(seq - (rel_slot >= 0 ? max(q_stamp, st_stamp) : q_stamp));
    // With a residual, the part this wave adds (its query group kh, the columns
    // its lanes finalise; rows past N read as zeros) is loaded now and lands
    // during the exchange.  Chunks of cut rows add it when they are combined.
    const bool add_r = RES && cur_row >= 0 && cur_slot < 0;
    v2u rres[NDT][4];
    if (add_r) {
      const __amdgpu_buffer_rsrc_t rrsc = make_rsrc(R + size_t(cur_bh) * size_t(N) * HD, head_bytes);
      const uint32_t rrow = uint32_t((cur_row - cur_bh * nb) * BLK + kh * 32 + ql) * W::ROWB;
#pragma unroll
      for (int u = 0; u < NDT; ++u)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          rres[u][g4] = __builtin_amdgcn_raw_buffer_load_b64(
              rrsc, rrow + uint32_t(32 * u + 8 * g4 + 4 * hh) * 2u, 0, 0);
    }
    // The previous epilogue's partial stores are complete: count them in.
    // (Only after a chunk of a cut row.  The count is read at once, on that
    // path alone: a wait for a memory result drains every load issued before
    // it, the next item's first tiles included, so the common path has none.)
    int mg_a = -1;
    if (rel_slot >= 0) {
      const int m = merge_of(rel_slot);
      if (m >= 0 && completes(m, __builtin_amdgcn_readfirstlane(count_in(m)))) mg_a = m;
      rel_slot = -1;
    }
    mg_a = __builtin_amdgcn_readfirstlane(mg_a);
    const bool more = k_nxt >= 0;
    lds_barrier();  // both halves of the staged query tile are in LDS
    if (more) read_q(qf);
    float l_half[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) l_half[g] = l_run[g] + other_half(l_run[g]);
    lds_barrier();  // the staging area is free for the exchange of m and l

    // Wave kh finalises query group kh; it sends its state of group 1 - kh
    // through the stage of its own ring that held the item's last tile (the
    // other holds the next item's first), and m, l through the staging area.
    // (Branches on kh keep every register array index a compile-time constant.)
    const int st_free = (ib + cur_cnt + 1) & 1;
    float* xml = reinterpret_cast<float*>(smem + 2 * size_t(W::RINGB));
    auto send = [&](const f32x16 (&a)[NDT], float m, float l) {
      float* xo = reinterpret_cast<float*>(smem + size_t(kh) * W::RINGB +
                                           size_t(st_free) * W::STAGEB);
#pragma unroll
      for (int u = 0; u < NDT; ++u)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<f32x4*>(xo + ((u * 4 + g4) * 64 + lane) * 4) =
              f32x4{a[u][4 * g4], a[u][4 * g4 + 1], a[u][4 * g4 + 2], a[u][4 * g4 + 3]};
      if (hh == 0) {
        xml[kh * 64 + ql] = m;
        xml[kh * 64 + 32 + ql] = l;
      }
    };
    int n_stores = 0;  // vector-memory stores this wave issues in the epilogue
    auto finish = [&](const f32x16 (&a)[NDT], float m0, float l0) {
      const int go = 1 - kh;
      const float* xi = reinterpret_cast<const float*>(smem + size_t(go) * W::RINGB +
                                                       size_t(st_free) * W::STAGEB);
      const float m1 = xml[go * 64 + ql];
      const float l1 = xml[go * 64 + 32 + ql];
      const float m = fmaxf(m0, m1);
      const float a0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - m);
      const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
      const float l = l0 * a0 + l1 * a1;
      f32x16 o[NDT];
#pragma unroll
      for (int u = 0; u < NDT; ++u)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 o1 = *reinterpret_cast<const f32x4*>(xi + ((u * 4 + g4) * 64 + lane) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[u][4 * g4 + e] = a[u][4 * g4 + e] * a0 + o1[e] * a1;
        }
      const int bh = cur_bh;
      const int q = kh * 32 + ql;
      const int qrow = (cur_row - bh * nb) * BLK + q;
      // Buffer stores with bounds: rows past N (and the lanes that carry no
      // m, l or LSE) address past the end and are dropped, so every wave
      // issues the same, known number of stores.
      if (cur_row >= 0 && cur_slot >= 0) {
        // Partial result of one chunk of a cut row (unnormalised acc, max in
        // log2 units, sum), combined with the row's other chunks by merge_kernel.
        constexpr uint32_t kSlotBytes = BLK * (HD + 2) * 4;
        const __amdgpu_buffer_rsrc_t pr = make_rsrc(part + size_t(cur_slot) * BLK * (HD + 2), kSlotBytes);
#pragma unroll
        for (int u = 0; u < NDT; ++u)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(v4u, f32x4{o[u][4 * g4], o[u][4 * g4 + 1], o[u][4 * g4 + 2],
                                              o[u][4 * g4 + 3]}),
                pr, uint32_t(q * HD + 32 * u + 8 * g4 + 4 * hh) * 4u, 0, kAgentScope);
        const float mw = m > kNoMax ? m : -INFINITY;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mw), pr,
                                              hh == 0 ? uint32_t(BLK * HD + q) * 4u : kSlotBytes, 0,
                                              kAgentScope);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l), pr,
                                              hh == 0 ? uint32_t(BLK * HD + BLK + q) * 4u : kSlotBytes,
                                              0, kAgentScope);
        n_stores = 4 * NDT + 2;
      } else if (cur_row >= 0) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const __amdgpu_buffer_rsrc_t orsc =
            make_rsrc(O + size_t(bh) * size_t(N) * HD, head_bytes);
        const uint32_t orow = uint32_t(qrow) * W::ROWB;
        // O = attention (+ R, summed in fp32), rounded once to bf16.
#pragma unroll
        for (int u = 0; u < NDT; ++u)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[u][i] *= inv;
        if (add_r) {
#pragma unroll
          for (int u = 0; u < NDT; ++u)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              o[u][4 * g4 + 0] += bf16_lo(rres[u][g4][0]);
              o[u][4 * g4 + 1] += bf16_hi(rres[u][g4][0]);
              o[u][4 * g4 + 2] += bf16_lo(rres[u][g4][1]);
              o[u][4 * g4 + 3] += bf16_hi(rres[u][g4][1]);
            }
        }
        // Lane (ql, hh) holds columns 32u + 8g4 + 4hh .. +3.  Swapping the odd-g4
        // pieces of the lower half-wave with the even-g4 pieces of the upper one
        // leaves every lane 8 contiguous columns (32u + 16p + 8hh .. +7), so four
        // 16-byte stores write the row.
#pragma unroll
        for (int u = 0; u < NDT; ++u)
#pragma unroll
          for (int pq = 0; pq < 2; ++pq) {
            const int ge = 2 * pq, go2 = 2 * pq + 1;
            const uint32_t e0 = pack_bf16x2(o[u][4 * ge + 0], o[u][4 * ge + 1]);
            const uint32_t e1 = pack_bf16x2(o[u][4 * ge + 2], o[u][4 * ge + 3]);
            const uint32_t d0v = pack_bf16x2(o[u][4 * go2 + 0], o[u][4 * go2 + 1]);
            const uint32_t d1v = pack_bf16x2(o[u][4 * go2 + 2], o[u][4 * go2 + 3]);
            // swap(X, Y): the upper lanes of the first result get the lower
            // lanes' Y, the lower lanes of the second result the upper lanes'
            // X.  Lower lanes need the upper half's even piece, upper lanes the
            // lower half's odd piece.
            const auto s0 = __builtin_amdgcn_permlane32_swap(e0, d0v, false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(e1, d1v, false, false);
            v4u w;
            if (hh == 0)
              w = v4u{e0, e1, s0[1], s1[1]};
            else
              w = v4u{s0[0], s1[0], d0v, d1v};
            __builtin_amdgcn_raw_buffer_store_b128(w, orsc, orow + uint32_t(32 * u + 16 * pq + 8 * hh) * 2u,
                                                   0, 0);
          }
        n_stores = 2 * NDT;
        if (LSE != nullptr) {
          const __amdgpu_buffer_rsrc_t lrsc =
              make_rsrc(LSE + size_t(bh) * size_t(N), static_cast<uint32_t>(N) * 4u);
          const float lv = l > 0.f ? (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lv), lrsc,
                                                hh == 0 ? uint32_t(qrow) * 4u : uint32_t(N) * 4u, 0, 0);
          n_stores = 2 * NDT + 1;
        }
      }
    };
    if (kh == 0)
      send(acc[1], m_run[1], l_half[1]);
    else
      send(acc[0], m_run[0], l_half[0]);
    // The item after next: the claim made one item ago (work list; wave 0
    // publishes its record through the staging area) or the next static round.
    int* xk = reinterpret_cast<int*>(xml + 128);
    if (queue && kh == 0) {
      if (claim_out && !nn_known) resolve_claim();  // an item without tiles
      if (lane == 0) {
        xk[0] = nn_k;
        xk[1] = nn_row;
        xk[2] = nn_c0;
        xk[3] = nn_cnt;
        xk[4] = nn_slot;
      }
    }
    lds_barrier();
    int k_nn;
    if (queue) {
      k_nn = xk[0];
      nn_row = xk[1];
      nn_c0 = xk[2];
      nn_cnt = xk[3];
      nn_slot = xk[4];
    } else {
      k_nn = src.stat(round);
    }
    int mg_b = -1;
    if (kh == 0)
      finish(acc[0], m_run[0], l_half[0]);
    else
      finish(acc[1], m_run[1], l_half[1]);
    lds_barrier();  // exchange areas free before loads target them again
    // Merges this wave completes: the previous chunk's (counted in above) and,
    // after the last item, this one's (its stores are waited for here).
    if (cur_row >= 0 && cur_slot >= 0) {
      if (more) {
        rel_slot = cur_slot;
      } else {
        const int m = merge_of(cur_slot);
        if (m >= 0) {
          wait_vm(0);
          if (completes(m, __builtin_amdgcn_readfirstlane(count_in(m)))) mg_b = m;
        }
      }
    }
    mg_b = __builtin_amdgcn_readfirstlane(mg_b);
    int merge_stores = 0;
    while (mg_a >= 0 || mg_b >= 0) {
      const int m = mg_a >= 0 ? mg_a : mg_b;
      if (mg_a >= 0)
        mg_a = -1;
      else
        mg_b = -1;
      merge_stores += merge_group(m);
    }
    merge_stores = __builtin_amdgcn_readfirstlane(merge_stores);
    seq += n_stores + merge_stores;
    st_stamp = seq;

    // ---- advance to the next item ------------------------------------------
    k_cur = k_nxt;
    k_nxt = k_nn;
    ++round;
    if (k_cur < 0) break;
    ib = (ib + cur_cnt) & 1;
    cur_row = nxt_row;
    cur_c0 = nxt_c0;
    cur_cnt = nxt_cnt;
    cur_slot = nxt_slot;
    cur_bh = nxt_bh;
    kd_cur = kd_nxt;
    vd_cur = vd_nxt;
    if (queue) {
      nxt_row = nn_row;
      nxt_c0 = nn_c0;
      nxt_cnt = nn_cnt;
      nxt_slot = nn_slot;
    } else {
      load_item(k_nxt, nxt_row, nxt_c0, nxt_cnt, nxt_slot);
    }
    nxt_bh = nxt_row >= 0 ? head_of(nxt_row) : 0;
    claim_out = queue && k_nxt >= 0;
    nn_known = false;
    nn_k = -1;
    nn_row = -1;
    nn_c0 = nn_cnt = 0;
    nn_slot = -1;
    if (claim_out && kh == 0) {
      if (lane == 0) ticket = src.claim(ctr);
      seq += 1;
    }
    kd_nxt = head_desc(K, nxt_row, nxt_bh);
    vd_nxt = head_desc(V, nxt_row, nxt_bh);
    stage_q(nxt_row, nxt_bh);
  }
  wait_vm(0);  // no load may still target LDS when the workgroup retires
}

// Gathered attention for token-level KV selection (page "Can sparse attention
// close the quality gap in diffusion transformers", section on token-level
// selection with tile-aligned query groups: KV tokens chosen one by one per query
// group and gathered by index, not repacked into blocks).  One workgroup of two
// wavefronts per (head, group of 64 queries): the queries of group g are the
// tokens groups[g][0..64), its keys and values the tokens tokens[g][0..T).  The
// tile formulation is the block forward's (S^T = K Q^T, wave h owns keys 32h..+31
// of every 64-token tile for all 64 queries); K operands and query rows are read
// straight from memory by index, each wave's 32 V rows pass through its own 4-KiB
// LDS area for the transposing reads.  O and LSE are written at the group's token
// positions.
constexpr int kGatherLds = 2 * 4096 + 2 * 8192 + 1024;  // V areas, key-half exchange, m and l

__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void gather_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const int32_t* __restrict__ groups,
    const int32_t* __restrict__ tokens, int32_t T, int32_t N, int32_t G, float sl2,
    uint16_t* __restrict__ O, float* __restrict__ LSE) {
  constexpr int HD = 64, ROWB = 128;
  __shared__ __align__(16) uint8_t smem[kGatherLds];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((BSA_LDS uint8_t*)smem));
  const int lane = threadIdx.x & 63;
  const int kh = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ql = lane & 31, hh = lane >> 5;
  const int row = blockIdx.x;
  const int bh = row / G;
  const int32_t* ids = groups + size_t(row) * 64;
  const int32_t* toks = tokens + size_t(row) * T;
  const uint32_t hbytes = static_cast<uint32_t>(N) * ROWB;
  const size_t head = size_t(bh) * size_t(N) * HD;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q + head, hbytes);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(K + head, hbytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(V + head, hbytes);
  const uint32_t vs = lds0 + uint32_t(kh) * 4096u;

  bf16x8 qf[2][4];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int t = ids[32 * g + ql];
    const uint32_t base = (t >= 0 && t < N) ? uint32_t(t) * ROWB : hbytes;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      qf[g][c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                qr, base + uint32_t(32 * c + 16 * hh), 0, 0));
  }
  float m_run[2] = {kNoMax, kNoMax}, l_run[2] = {0.f, 0.f};
  f32x16 acc[2][2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[g][u][i] = 0.f;

  // Token of this lane's key at list position idx (-1 past the list or out of range).
  auto tok_at = [&](int idx) {
    const int t = idx < T ? toks[idx] : -1;
    return (t >= 0 && t < N) ? t : -1;
  };
  // K operand of this lane's key and the V chunks this lane stages (row r = 8i +
  // lane / 8 of the wave's 32 keys, 16-byte chunk lane % 8); the V rows' tokens
  // come from the lanes that hold those keys.
  auto load_tile = [&](int ktok, bf16x8 (&ka)[4], v4u (&vx)[4]) {
    const uint32_t kbase = ktok >= 0 ? uint32_t(ktok) * ROWB : hbytes;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      ka[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                             kr, kbase + uint32_t(32 * c + 16 * hh), 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * i + (lane >> 3);
      const int vt = __builtin_amdgcn_ds_bpermute(r << 2, ktok);
      const uint32_t vb = vt >= 0 ? uint32_t(vt) * ROWB : hbytes;
      vx[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, vb + uint32_t(16 * (lane & 7)), 0, 0);
    }
  };
  // One 64-key tile: S^T for this wave's 32 keys (K operand ka, token ktok of the
  // lane's key), online softmax, then P V with the V rows vx staged in LDS.
  auto tile = [&](int ktok, const bf16x8 (&ka)[4], const v4u (&vx)[4]) {
    // Keys of this wave's half of the tile that exist (bit j: key 32 kh + j).
    const uint32_t kvalid = static_cast<uint32_t>(__builtin_amdgcn_ballot_w64(ktok >= 0));
    const f32x16 zero = {};
    f32x16 s[2];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int g = 0; g < 2; ++g)
        s[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qf[g][c], c == 0 ? zero : s[g], 0, 0, 0);
    // Keys past the list (or out of range) get -inf.
    if (kvalid != 0xffffffffu) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!((kvalid >> (8 * (i >> 2) + 4 * hh + (i & 3))) & 1u)) {
          s[0][i] = -INFINITY;
          s[1][i] = -INFINITY;
        }
    }
    bf16x8 pb[2][2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float mx = vmax(s[g][0], s[g][1]);
#pragma unroll
      for (int i = 2; i < 16; ++i) mx = vmax(mx, s[g][i]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = vmax(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const float mt = vmax(m_run[g], mx * sl2);
      const float alpha = __builtin_amdgcn_exp2f(m_run[g] - mt);
      l_run[g] *= alpha;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][u][i] *= alpha;
      m_run[g] = mt;
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[g][i], sl2, -mt));
        ls += p;
        pb[g][i >> 3][i & 7] = static_cast<__bf16>(p);
      }
      l_run[g] += ls;
    }
    // This tile's V rows into the wave's LDS area (the previous tile's reads are
    // done: one wavefront's LDS operations complete in order).
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<BSA_LDS v4u*>(static_cast<uintptr_t>(vs + swz<ROWB>(8 * i + (lane >> 3), lane & 7))) = vx[i];
    const int tr_row = 4 * hh + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int u2 = 0; u2 < 2; ++u2) {
        const int col = 32 * u2 + tr_col;
        const v4s lo = lds_read_tr(vs + swz<ROWB>(16 * c2 + tr_row, col >> 3) + (col & 7) * 2);
        const v4s hi = lds_read_tr(vs + swz<ROWB>(16 * c2 + 8 + tr_row, col >> 3) + (col & 7) * 2);
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int g = 0; g < 2; ++g)
          acc[g][u2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[g][c2], acc[g][u2], 0, 0, 0);
      }
  };
  // Two K/V register sets in turn: the next tile's rows are in flight while a
  // tile is computed, and the token indices one tile further ahead.  Loads for
  // tiles past the list use out-of-range offsets (zeros, no memory traffic).
  const int ntiles = (T + 63) / 64;
  int t_cur = tok_at(32 * kh + ql), t_next = tok_at(64 + 32 * kh + ql);
  bf16x8 ka0[4], ka1[4];
  v4u vx0[4], vx1[4];
  load_tile(t_cur, ka0, vx0);
  for (int tt = 0; tt < ntiles; tt += 2) {
    {
      const int t_nn = tok_at(64 * (tt + 2) + 32 * kh + ql);
      load_tile(t_next, ka1, vx1);
      tile(t_cur, ka0, vx0);
      t_cur = t_next;
      t_next = t_nn;
    }
    if (tt + 1 < ntiles) {
      const int t_nn = tok_at(64 * (tt + 3) + 32 * kh + ql);
      load_tile(t_next, ka0, vx0);
      tile(t_cur, ka1, vx1);
      t_cur = t_next;
      t_next = t_nn;
    }
  }

  // Key-half merge: wave kh finalises query group kh; it sends its state of group
  // 1 - kh through the exchange area.
  float l_half[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) l_half[g] = l_run[g] + other_half(l_run[g]);
  float* xo_base = reinterpret_cast<float*>(smem + 8192);
  float* xml = reinterpret_cast<float*>(smem + 8192 + 16384);
  auto send = [&](const f32x16 (&a)[2], float m, float l) {
    float* xo = xo_base + size_t(kh) * 2048;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<f32x4*>(xo + ((u * 4 + g4) * 64 + lane) * 4) =
            f32x4{a[u][4 * g4], a[u][4 * g4 + 1], a[u][4 * g4 + 2], a[u][4 * g4 + 3]};
    if (hh == 0) {
      xml[kh * 64 + ql] = m;
      xml[kh * 64 + 32 + ql] = l;
    }
  };
  auto finish = [&](const f32x16 (&a)[2], float m0, float l0) {
    const int go = 1 - kh;
    const float* xi = xo_base + size_t(go) * 2048;
    const float m1 = xml[go * 64 + ql], l1 = xml[go * 64 + 32 + ql];
    const float m = fmaxf(m0, m1);
    const float a0 = m0 <= kNoMax ? 0.f : __builtin_amdgcn_exp2f(m0 - m);
    const float a1 = m1 <= kNoMax ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
    const float l = l0 * a0 + l1 * a1;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int t = ids[32 * kh + ql];
    const bool ok = t >= 0 && t < N;
    uint16_t* orow = O + head + size_t(ok ? t : 0) * HD;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(xi + ((u * 4 + g4) * 64 + lane) * 4);
        if (ok) {
          const int d = 32 * u + 8 * g4 + 4 * hh;
          const uint32_t w0 = pack_bf16x2((a[u][4 * g4] * a0 + o1[0] * a1) * inv,
                                          (a[u][4 * g4 + 1] * a0 + o1[1] * a1) * inv);
          const uint32_t w1 = pack_bf16x2((a[u][4 * g4 + 2] * a0 + o1[2] * a1) * inv,
                                          (a[u][4 * g4 + 3] * a0 + o1[3] * a1) * inv);
          *reinterpret_cast<uint2*>(orow + d) = make_uint2(w0, w1);
        }
      }
    if (LSE != nullptr && ok && hh == 0)
      LSE[size_t(bh) * N + t] = l > 0.f ? (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
  };
  if (kh == 0)
    send(acc[1], m_run[1], l_half[1]);
  else
    send(acc[0], m_run[0], l_half[0]);
  __syncthreads();
  if (kh == 0)
    finish(acc[0], m_run[0], l_half[0]);
  else
    finish(acc[1], m_run[1], l_half[1]);
}

// Combines the chunk partials of every cut row: with M = max_c m_c,
// O = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c and LSE = (M + log2 L) ln 2.
// One thread per (query row, 4 output columns); the loads of up to kUnroll
// chunks are issued together, so a merge costs about one memory round trip.
constexpr int kMergeThreads = 256;
constexpr int kUnroll = 8;

// Gathered attention at head dim 128 (same page and section as gather_kernel).
// One workgroup of four wavefronts per (head, group of 64 queries): wave w owns
// query group w % 2 (32 of the group's queries) and key half w / 2 (keys
// 32 (w / 2) .. +31 of every 64-token tile).  The tile's 64 K and V rows are
// gathered by token index into registers one tile ahead (every lane moves
// eight 16-byte chunks: rows 4 (w + 4 s) + lane / 16, s = 0..3, of K and of V)
// and written to LDS, swizzled, in two stages; one barrier per tile makes the
// rows visible and frees the other stage.  The compute is the block forward's
// at D = 128: S^T = K Q^T with the K operands from LDS, the online softmax,
// O^T += V^T P^T with V^T read transposed; the key halves meet at the end
// through LDS and O, LSE are written at the group's token positions.
struct Gather128 {
  static constexpr int HD = 128, ROWB = 256, TILEB = 64 * ROWB;  // 16 KiB
  static constexpr int STAGEB = 2 * TILEB;                         // K tile, V tile
  static constexpr size_t LDS_BYTES = 2 * STAGEB + 2 * 64 * 2 * 4;  // + m, l exchange
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gather128_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const int32_t* __restrict__ groups,
    const int32_t* __restrict__ tokens, int32_t T, int32_t N, int32_t G, float sl2,
    uint16_t* __restrict__ O, float* __restrict__ LSE) {
  using GC = Gather128;
  constexpr int HD = GC::HD, ROWB = GC::ROWB;
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((BSA_LDS uint8_t*)smem));
  float* ml = reinterpret_cast<float*>(smem + 2 * size_t(GC::STAGEB));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qg = wave & 1, kh = wave >> 1;
  const int ql = lane & 31, hh = lane >> 5;
  const int row = blockIdx.x;
  const int bh = row / G;
  const int32_t* ids = groups + size_t(row) * 64;
  const int32_t* toks = tokens + size_t(row) * T;
  const uint32_t hbytes = static_cast<uint32_t>(N) * ROWB;
  const size_t head = size_t(bh) * size_t(N) * HD;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q + head, hbytes);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(K + head, hbytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(V + head, hbytes);

  // Query fragments (B operand of S^T = K Q^T): d = 16c + 8hh .. +7 of query
  // ids[32 qg + ql]; a query outside [0, N) reads zeros.
  bf16x8 qf[8];
  {
    const int t = ids[32 * qg + ql];
    const uint32_t base = (t >= 0 && t < N) ? uint32_t(t) * ROWB : hbytes;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      qf[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                             qr, base + uint32_t(32 * c + 16 * hh), 0, 0));
  }
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[u][i] = 0.f;

  // Token at list position idx, or -1 past the list or outside [0, N).
  auto tok_at = [&](int idx) {
    const int t = idx < T ? toks[idx] : -1;
    return (t >= 0 && t < N) ? t : -1;
  };
  // This lane's chunks of tile tt: K and V rows 4 (wave + 4 sg) + lane / 16
  // (sg = 0..3: the 16 1-KiB segments of a tile over the four waves), chunk
  // lane % 16 of each row's LDS position, from source chunk
  // (lane % 16) ^ swizzle(row).  ltok: the lane's token of the tile (lane l
  // holds position l).
  v4u kx[4], vx[4];
  auto load_rows = [&](int ltok) {
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) {
      const int r = 4 * (wave + 4 * sg) + (lane >> 4);
      const int t = __builtin_amdgcn_ds_bpermute(r << 2, ltok);
      const uint32_t src = t >= 0 ? uint32_t(t) * ROWB + uint32_t(((lane & 15) ^
                                        chunk_swizzle<ROWB>(r)) << 4)
                                  : hbytes;
      kx[sg] = __builtin_amdgcn_raw_buffer_load_b128(kr, src, 0, 0);
      vx[sg] = __builtin_amdgcn_raw_buffer_load_b128(vr, src, 0, 0);
    }
  };
  auto store_rows = [&](int st) {
    const uint32_t kb = lds0 + uint32_t(st) * GC::STAGEB;
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) {
      const uint32_t off = uint32_t(wave + 4 * sg) * 1024u + uint32_t(lane) * 16u;
      *reinterpret_cast<BSA_LDS v4u*>(static_cast<uintptr_t>(kb + off)) = kx[sg];
      *reinterpret_cast<BSA_LDS v4u*>(static_cast<uintptr_t>(kb + GC::TILEB + off)) = vx[sg];
    }
  };

  const int ntiles = (T + 63) / 64;
  int ltok = tok_at(lane);
  load_rows(ltok);
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  for (int tt = 0; tt < ntiles; ++tt) {
    const int st = tt & 1;
    // Keys of this wave's half that exist (bit j: key 32 kh + j of the tile).
    const uint32_t kvalid =
        static_cast<uint32_t>(__builtin_amdgcn_ballot_w64(ltok >= 0) >> (32 * kh));
    store_rows(st);  // the other waves finished reading this stage (tile tt - 2)
    if (tt + 1 < ntiles) {
      ltok = tok_at(64 * (tt + 1) + lane);
      load_rows(ltok);
    }
    __syncthreads();  // tile tt is in LDS; every wave is done with tile tt - 1
    const uint32_t ks = lds0 + uint32_t(st) * GC::STAGEB, vs = ks + GC::TILEB;
    const int key = 32 * kh + ql;
    bf16x8 ka[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) ka[c] = lds_read16(ks + swz<ROWB>(key, 2 * c + hh));
    const f32x16 zero = {};
    f32x16 sv = zero;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qf[c], c == 0 ? zero : sv, 0, 0, 0);
    v4s vlo[2][4], vhi[2][4];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int u2 = 0; u2 < 4; ++u2) {
        const int kb = 32 * kh + 16 * c2;
        const int col = 32 * u2 + tr_col;
        vlo[c2][u2] = lds_read_tr(vs + swz<ROWB>(kb + tr_row, col >> 3) + (col & 7) * 2);
        vhi[c2][u2] = lds_read_tr(vs + swz<ROWB>(kb + 8 + tr_row, col >> 3) + (col & 7) * 2);
      }
    // register i: key 8(i/4) + 4hh + (i%4) of this half; missing keys get -inf
    if (kvalid != 0xffffffffu) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!((kvalid >> (8 * (i >> 2) + 4 * hh + (i & 3))) & 1u)) sv[i] = -INFINITY;
    }
    float mx = sv[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[i]);
    mx = fmaxf(mx, other_half(mx));
    const float mt = fmaxf(m_run, mx * sl2);
    const float alpha = m_run == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - mt);
    l_run *= alpha;
#pragma unroll
    for (int u2 = 0; u2 < 4; ++u2)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[u2][i] *= alpha;
    m_run = mt;
    const float m_use = mt == -INFINITY ? 0.f : mt;
    bf16x8 pb[2];
    float ls[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sv[i], sl2, -m_use));
      if (i < 4)
        ls[i] = p;
      else
        ls[i & 3] += p;
      pb[i >> 3][i & 7] = static_cast<__bf16>(p);
    }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int u2 = 0; u2 < 4; ++u2) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(vlo[c2][u2], vhi[c2][u2], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[u2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c2], acc[u2], 0, 0, 0);
      }
  }

  // Key-half merge through stage 0 (every wave is past its last tile's reads
  // once all have arrived): wave (qg, 1) sends its state, wave (qg, 0) combines
  // and writes the group's rows.
  const float l_half = l_run + other_half(l_run);
  __syncthreads();
  float* mg = reinterpret_cast<float*>(smem) + size_t(qg) * 64 * 4 * 16;
  if (kh == 1) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<f32x4*>(mg + ((u * 4 + g4) * 64 + lane) * 4) =
            f32x4{acc[u][4 * g4], acc[u][4 * g4 + 1], acc[u][4 * g4 + 2], acc[u][4 * g4 + 3]};
    ml[(qg * 2) * 64 + lane] = m_run;
    ml[(qg * 2 + 1) * 64 + lane] = l_half;
  }
  __syncthreads();
  if (kh == 0) {
    const float m1 = ml[(qg * 2) * 64 + lane];
    const float l1 = ml[(qg * 2 + 1) * 64 + lane];
    const float m = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
    const float l = l_half * a0 + l1 * a1;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int t = ids[32 * qg + ql];
    if (t >= 0 && t < N) {
      uint16_t* orow = O + head + size_t(t) * HD;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 o1 = *reinterpret_cast<const f32x4*>(mg + ((u * 4 + g4) * 64 + lane) * 4);
          const int d = 32 * u + 8 * g4 + 4 * hh;
          const uint32_t w0 = pack_bf16x2((acc[u][4 * g4] * a0 + o1[0] * a1) * inv,
                                          (acc[u][4 * g4 + 1] * a0 + o1[1] * a1) * inv);
          const uint32_t w1 = pack_bf16x2((acc[u][4 * g4 + 2] * a0 + o1[2] * a1) * inv,
                                          (acc[u][4 * g4 + 3] * a0 + o1[3] * a1) * inv);
          *reinterpret_cast<uint2*>(orow + d) = make_uint2(w0, w1);
        }
      if (LSE != nullptr && hh == 0)
        LSE[size_t(bh) * N + t] =
            l > 0.f ? (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
    }
  }
}

template <int BLK, int HD, bool RES>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const int32_t* __restrict__ merges,
                                                              const float* __restrict__ part,
                                                              int32_t N, int32_t nb,
                                                              int32_t n_rows,
                                                              uint16_t* __restrict__ O,
                                                              float* __restrict__ LSE,
                                                              const uint16_t* __restrict__ R) {
  constexpr int D4 = HD / 4;
  constexpr int WG_PER_ROW = BLK * D4 / kMergeThreads;
  constexpr size_t SLOT = size_t(BLK) * (HD + 2);
  const int m = blockIdx.x / WG_PER_ROW;
  const int idx = (blockIdx.x - m * WG_PER_ROW) * kMergeThreads + threadIdx.x;
  const int r = merges[3 * m], slot0 = merges[3 * m + 1], nch = merges[3 * m + 2];
  if (r < 0 || r >= n_rows || nch < 1) return;
  const int bh = r / nb;
  const int q = idx / D4;
  const int d = (idx - q * D4) * 4;
  const int qrow = (r - bh * nb) * BLK + q;
  if (qrow >= N) return;
  const float* base = part + size_t(slot0) * SLOT;

  float mc[kUnroll], lc[kUnroll];
  f32x4 oc[kUnroll];
  const int n0 = min(nch, kUnroll);
#pragma unroll
  for (int c = 0; c < kUnroll; ++c) {
    if (c < n0) {
      const float* pc = base + size_t(c) * SLOT;
      mc[c] = pc[BLK * HD + q];
      lc[c] = pc[BLK * HD + BLK + q];
      oc[c] = *reinterpret_cast<const f32x4*>(pc + q * HD + d);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int c = 0; c < kUnroll; ++c)
    if (c < n0) M = fmaxf(M, mc[c]);
  for (int c = kUnroll; c < nch; ++c) M = fmaxf(M, base[size_t(c) * SLOT + BLK * HD + q]);
  float L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
#pragma unroll
    for (int c = 0; c < kUnroll; ++c) {
      if (c < n0) {
        const float w = mc[c] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc[c] - M);
        L += w * lc[c];
        o += w * oc[c];
      }
    }
    for (int c = kUnroll; c < nch; ++c) {
      const float* pc = base + size_t(c) * SLOT;
      const float mm = pc[BLK * HD + q];
      const float w = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mm - M);
      L += w * pc[BLK * HD + BLK + q];
      o += w * *reinterpret_cast<const f32x4*>(pc + q * HD + d);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const size_t head = size_t(bh) * size_t(N) * HD;
  f32x4 y = o * inv;
  if (RES) {  // O = attention + R, summed in fp32, rounded once
    const uint2 rv = *reinterpret_cast<const uint2*>(R + head + size_t(qrow) * HD + d);
    y += f32x4{bf16_lo(rv.x), bf16_hi(rv.x), bf16_lo(rv.y), bf16_hi(rv.y)};
  }
  *reinterpret_cast<uint2*>(O + head + size_t(qrow) * HD + d) =
      make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
  if (d == 0 && LSE != nullptr)
    LSE[size_t(bh) * N + qrow] =
        L > 0.f ? (M + __builtin_amdgcn_logf(L)) * 0.69314718055994531f : -INFINITY;
}

// Resident workgroups of fwd_kernel<BLK, HD, RES> on the current device (cached).
template <int BLK, int HD, bool RES>
int resident_workgroups() {
  using C = FwdCfg<BLK, HD>;
  static std::once_flag once;
  static int n = 0;
  std::call_once(once, [] {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&fwd_kernel<BLK, HD, RES>), C::NT,
            C::LDS_BYTES) != hipSuccess)
      return;
    n = cus * (per_cu > 0 ? per_cu : 1);
  });
  return n;
}

// Workgroups to launch for `items` items with `resident` resident slots.  With
// a work list every group needs at least one workgroup, so the grid never
// drops below BSA_MAX_GROUPS (workgroups without an item leave at once).
int32_t launch_grid(int32_t items, int resident, bool queued) {
  if (items <= 0) return 0;
  int32_t g = items < resident ? items : resident;
  if (queued && g < BSA_MAX_GROUPS) g = BSA_MAX_GROUPS;
  return g;
}

template <int HD, bool RES>
int resident_wide_workgroups() {
  static std::once_flag once;
  static int n = 0;
  std::call_once(once, [] {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&fwd_wide_kernel<HD, RES>), Wide<HD>::NT,
            Wide<HD>::LDS_BYTES) != hipSuccess)
      return;
    n = cus * (per_cu > 0 ? per_cu : 1);
  });
  return n;
}

template <int HD, bool RES>
bsa_status launch_wide(const void* q, const void* k, const void* v, int32_t N, int32_t nb,
                       int32_t n_rows, const int32_t* row_ptr, const int32_t* col_idx,
                       const int32_t* work, int32_t n_items, int32_t n_merges, int32_t n_slots,
                       float sl2, void* o, float* lse, float* part, int32_t* ctr, int32_t* mctr,
                       const void* r, hipStream_t stream) {
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_wide_kernel<HD, RES>),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(Wide<HD>::LDS_BYTES));
  });
  if (attr != hipSuccess) return BSA_ERR_HIP;
  const int32_t items = work ? n_items : n_rows;
  const int resident = resident_wide_workgroups<HD, RES>();
  if (resident <= 0) return BSA_ERR_HIP;
  const int32_t grid = launch_grid(items, resident, work != nullptr);
  if (grid > 0) {
    hipLaunchKernelGGL((fwd_wide_kernel<HD, RES>), dim3(grid), dim3(Wide<HD>::NT), Wide<HD>::LDS_BYTES, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), row_ptr, col_idx, work, items, n_merges,
                       N, nb, n_rows, sl2, static_cast<uint16_t*>(o), lse, part, ctr,
                       work ? n_slots : 0, mctr, static_cast<const uint16_t*>(r));
    BSA_HIP_CHECK_LAUNCH();
  }
  return BSA_OK;
}

template <int BLK, int HD, bool RES>
bsa_status launch_fwd(const void* q, const void* k, const void* v, int32_t N, int32_t nb,
                      int32_t n_rows, const int32_t* row_ptr, const int32_t* col_idx,
                      const int32_t* work, int32_t n_items, int32_t n_merges, float sl2, void* o,
                      float* lse, float* part, int32_t* ctr, const void* r, hipStream_t stream) {
  using C = FwdCfg<BLK, HD>;
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_kernel<BLK, HD, RES>),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(C::LDS_BYTES));
  });
  if (attr != hipSuccess) return BSA_ERR_HIP;
  const int32_t items = work ? n_items : n_rows;
  const int resident = resident_workgroups<BLK, HD, RES>();
  if (resident <= 0) return BSA_ERR_HIP;
  const int32_t grid = launch_grid(items, resident, work != nullptr);
  if (grid > 0) {
    hipLaunchKernelGGL((fwd_kernel<BLK, HD, RES>), dim3(grid), dim3(C::NT), C::LDS_BYTES, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), row_ptr, col_idx, work, items, n_merges,
                       N, nb, n_rows, sl2, static_cast<uint16_t*>(o), lse, part, ctr,
                       static_cast<const uint16_t*>(r));
    BSA_HIP_CHECK_LAUNCH();
  }
  if (work && n_merges > 0) {
    constexpr int wg_per_row = BLK * (HD / 4) / kMergeThreads;
    hipLaunchKernelGGL((merge_kernel<BLK, HD, RES>), dim3(n_merges * wg_per_row), dim3(kMergeThreads),
                       0, stream,
                       work + 4 * size_t(n_items), part, N, nb, n_rows,
                       static_cast<uint16_t*>(o), lse, static_cast<const uint16_t*>(r));
    BSA_HIP_CHECK_LAUNCH();
  }
  return BSA_OK;
}

}  // namespace
}  // namespace bsa

extern "C" BSA_API size_t bsa_forward_workspace_bytes(int32_t n_slots, int32_t D,
                                                      int32_t block) {
  if (n_slots < 0 || D < 1 || block < 1) return 0;
  return bsa::kCounterBytes + bsa::merge_counter_bytes(n_slots) +
         size_t(n_slots) * size_t(block) * size_t(D + 2) * sizeof(float);
}

namespace bsa {
namespace {
// The forward with an optional residual r added before O is rounded.
bsa_status forward_impl(const void* q, const void* k, const void* v, int32_t B, int32_t H,
                        int32_t N, int32_t D, int32_t block, const int32_t* row_ptr_dev,
                        const int32_t* col_idx_dev, const int32_t* work_dev, int32_t n_items,
                        int32_t n_merges, int32_t n_slots, float scale, const void* r, void* o,
                        float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !row_ptr_dev || !col_idx_dev) return BSA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return BSA_ERR_INVALID_ARG;
  if (!supported_shape(D, block)) return BSA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return BSA_ERR_INVALID_ARG;
  if (r != nullptr && !aligned16(r)) return BSA_ERR_INVALID_ARG;
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
    if (!workspace || !aligned16(workspace)) return BSA_ERR_INVALID_ARG;
    if (workspace_bytes < bsa_forward_workspace_bytes(n_slots, D, block)) return BSA_ERR_CAPACITY;
  } else {
    n_items = n_merges = 0;
  }
  const float sc = scale > 0.f ? scale : 1.f / sqrtf(static_cast<float>(D));
  const float sl2 = sc * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* ctr = work_dev ? static_cast<int32_t*>(workspace) : nullptr;
  int32_t* mctr = work_dev ? reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) +
                                                        kCounterBytes)
                           : nullptr;
  float* part = work_dev ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                                    kCounterBytes + merge_counter_bytes(n_slots))
                         : nullptr;
#define BSA_FWD_ARGS                                                                            \
  q, k, v, N, nb, n_rows, row_ptr_dev, col_idx_dev, work_dev, n_items, n_merges, sl2, o, lse, \
      part, ctr, r, s
  const bool res = r != nullptr;
#define BSA_WIDE_ARGS                                                                           \
  q, k, v, N, nb, n_rows, row_ptr_dev, col_idx_dev, work_dev, n_items, n_merges, n_slots, sl2, o, \
      lse, part, ctr, mctr, r, s
  if (block == 64 && D == 64)
    return res ? launch_wide<64, true>(BSA_WIDE_ARGS) : launch_wide<64, false>(BSA_WIDE_ARGS);
  if (block == 64 && D == 128)
    return res ? launch_wide<128, true>(BSA_WIDE_ARGS) : launch_wide<128, false>(BSA_WIDE_ARGS);
#undef BSA_WIDE_ARGS
  if (block == 128 && D == 64)
    return res ? launch_fwd<128, 64, true>(BSA_FWD_ARGS) : launch_fwd<128, 64, false>(BSA_FWD_ARGS);
  return res ? launch_fwd<128, 128, true>(BSA_FWD_ARGS) : launch_fwd<128, 128, false>(BSA_FWD_ARGS);
#undef BSA_FWD_ARGS
}
}  // namespace
}  // namespace bsa

extern "C" BSA_API bsa_status bsa_forward(const void* q, const void* k, const void* v,
                                          int32_t B, int32_t H, int32_t N, int32_t D,
                                          int32_t block, const int32_t* row_ptr_dev,
                                          const int32_t* col_idx_dev, const int32_t* work_dev,
                                          int32_t n_items, int32_t n_merges, int32_t n_slots,
                                          float scale, void* o, float* lse, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  return bsa::forward_impl(q, k, v, B, H, N, D, block, row_ptr_dev, col_idx_dev, work_dev,
                           n_items, n_merges, n_slots, scale, nullptr, o, lse, workspace,
                           workspace_bytes, stream);
}

extern "C" BSA_API bsa_status bsa_forward_compensated(
    const void* q, const void* k, const void* v, int32_t B, int32_t H, int32_t N, int32_t D,
    int32_t block, const int32_t* row_ptr_dev, const int32_t* col_idx_dev,
    const int32_t* work_dev, int32_t n_items, int32_t n_merges, int32_t n_slots, float scale,
    const void* r, void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (r == nullptr) return BSA_ERR_INVALID_ARG;
  // r and o must not overlap (r is read while other rows of o are written).
  const size_t bytes = size_t(B > 0 ? B : 0) * size_t(H > 0 ? H : 0) * size_t(N > 0 ? N : 0) *
                       size_t(D > 0 ? D : 0) * 2;
  const uintptr_t rb = reinterpret_cast<uintptr_t>(r), ob = reinterpret_cast<uintptr_t>(o);
  if (o != nullptr && rb < ob + bytes && ob < rb + bytes) return BSA_ERR_INVALID_ARG;
  return bsa::forward_impl(q, k, v, B, H, N, D, block, row_ptr_dev, col_idx_dev, work_dev,
                           n_items, n_merges, n_slots, scale, r, o, lse, workspace,
                           workspace_bytes, stream);
}

extern "C" BSA_API bsa_status bsa_gather_forward(const void* q, const void* k, const void* v,
                                                 int32_t B, int32_t H, int32_t N, int32_t D,
                                                 const int32_t* groups, int32_t G,
                                                 const int32_t* tokens, int32_t T, float scale,
                                                 void* o, float* lse, void* stream) {
  using namespace bsa;
  if (!q || !k || !v || !o || !groups || (!tokens && T > 0)) return BSA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || G < 1 || T < 0 || !(scale == scale)) return BSA_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return BSA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return BSA_ERR_INVALID_ARG;
  if (int64_t(N) * D * 2 >= (int64_t(1) << 31) || int64_t(B) * H * G > INT32_MAX) return BSA_ERR_UNSUPPORTED;
  const float sc = scale > 0.f ? scale : 1.f / sqrtf(static_cast<float>(D));
  if (D == 128) {
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
      attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gather128_kernel),
                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                 static_cast<int>(Gather128::LDS_BYTES));
    });
    if (attr != hipSuccess) return BSA_ERR_HIP;
    hipLaunchKernelGGL(gather128_kernel, dim3(B * H * G), dim3(256), Gather128::LDS_BYTES,
                       static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), groups,
                       tokens, T, N, G, sc * 1.4426950408889634f, static_cast<uint16_t*>(o), lse);
    BSA_HIP_CHECK_LAUNCH();
    return BSA_OK;
  }
  hipLaunchKernelGGL(gather_kernel, dim3(B * H * G), dim3(128), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), groups, tokens, T, N, G,
                     sc * 1.4426950408889634f, static_cast<uint16_t*>(o), lse);
  BSA_HIP_CHECK_LAUNCH();
  return BSA_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free forward: the work-list workspace lives in a static device
// array instead of a caller buffer.
namespace bsa {
namespace {

// Largest workspace bsa_forward_noalloc serves: the item counters (256 KiB),
// the merge counters and the partial results of cut rows.
constexpr size_t kNoAllocScratchBytes = BSA_FORWARD_NOALLOC_MAX_BYTES;
static_assert(kNoAllocScratchBytes == (size_t(16) << 20), "header and library agree");
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// Device address of `scratch` per device, taken once per device with that
// device current (the host-side name of the array is not a device address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

bsa_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return BSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return BSA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BSA_OK;
}

// Zeroes the item counters (one per group, kCounterStride apart) and the
// merge counters that follow them.
__global__ __launch_bounds__(256) void clear_counters_kernel(int32_t* __restrict__ ctr,
                                                             int32_t n_merge_ints) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < BSA_MAX_GROUPS) ctr[size_t(t) * kCounterStride] = 0;
  int32_t* mctr = ctr + kCounterBytes / sizeof(int32_t);
  if (t < n_merge_ints) mctr[t] = 0;
}

}  // namespace
}  // namespace bsa

extern "C" BSA_API bsa_status bsa_forward_noalloc(const void* q, const void* k, const void* v,
                                                  int32_t B, int32_t H, int32_t N, int32_t D,
                                                  int32_t block, const int32_t* row_ptr_dev,
                                                  const int32_t* col_idx_dev,
                                                  const int32_t* work_dev, int32_t n_items,
                                                  int32_t n_merges, int32_t n_slots, float scale,
                                                  void* o, float* lse, void* stream) {
  using namespace bsa;
  if (!work_dev)
    return bsa_forward(q, k, v, B, H, N, D, block, row_ptr_dev, col_idx_dev, nullptr, 0, 0, 0,
                       scale, o, lse, nullptr, 0, stream);
  if (n_slots < 0 || D < 1 || block < 1) return BSA_ERR_INVALID_ARG;
  const size_t need = bsa_forward_workspace_bytes(n_slots, D, block);
  if (need == 0 || need > kNoAllocScratchBytes) return BSA_ERR_CAPACITY;
  // Argument checks before anything is enqueued (bsa_forward repeats them).
  if (!q || !k || !v || !o || !row_ptr_dev || !col_idx_dev) return BSA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || n_items < 0 || n_merges < 0) return BSA_ERR_INVALID_ARG;
  if (!supported_shape(D, block)) return BSA_ERR_UNSUPPORTED;
  void* ws = nullptr;
  const bsa_status st = scratch_of_current_device(&ws);
  if (st != BSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t n_merge_ints = static_cast<int32_t>(merge_counter_bytes(n_slots) / sizeof(int32_t));
  const int32_t n_clear = n_merge_ints > BSA_MAX_GROUPS ? n_merge_ints : BSA_MAX_GROUPS;
  hipLaunchKernelGGL(clear_counters_kernel, dim3((n_clear + 255) / 256), dim3(256), 0, s,
                     static_cast<int32_t*>(ws), n_merge_ints);
  BSA_HIP_CHECK_LAUNCH();
  return bsa_forward(q, k, v, B, H, N, D, block, row_ptr_dev, col_idx_dev, work_dev, n_items,
                     n_merges, n_slots, scale, o, lse, ws, kNoAllocScratchBytes, stream);
}
