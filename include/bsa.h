/*
 * bsa.h - C ABI of libbsa: block-sparse FlashAttention forward and its
 * mean-pool top-k block-mask builder, for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages; cited by title and section):
 *   BSA-DiT   "多模态DiT中的块稀疏注意力：从原理到工程落地" (block-sparse attention
 *             in multimodal DiTs, from principle to deployment), m.nlpx.cn.
 *   MC-Sparse summary  "Can sparse attention close the quality gap in
 *             diffusion transformers" (wispaper.ai summary of the MC-Sparse paper).
 *
 * Conventions shared by every entry point
 *   - Q, K, V, O: bf16, contiguous [B, H, N, D] (D fastest), 16-byte aligned.
 *   - block size b is both the query-block and the KV-block size; nb = ceil(N/b).
 *     The last block may be partial: its missing query rows are neither
 *     computed nor stored, its missing keys are masked out.
 *   - CSR row r = (bi*H + h)*nb + i lists the KV blocks that query block i of
 *     head (bi, h) attends to: row_ptr int32 [B*H*nb + 1], col_idx int32 [nnz],
 *     nnz = row_ptr[B*H*nb].  Columns of a row are in [0, nb) and distinct: a
 *     block is either active or not (BSA-DiT §4.1, §4.3), while the forward
 *     would count the keys of a repeated column twice.  The mask builder writes
 *     them strictly ascending; the forward needs no order.
 *     bsa_validate_csr_host checks both (strict = 1) or distinctness alone (2).
 *   - LSE: fp32 [B, H, N], natural log, including the softmax scale.
 *   - Supported: D in {64, 128}, b in {64, 128}, 1 <= N, nb <= 1024.
 *   - Ownership: the caller allocates every buffer (device buffers with
 *     hipMalloc or torch, host buffers anywhere); the library allocates no
 *     memory and keeps no state (bsa_forward_noalloc aside: its static device
 *     array and that array's address per device).  Device work is enqueued on `stream`
 *     (a hipStream_t passed as void*; NULL = the null stream) and is
 *     asynchronous: the library never synchronises.
 *   - Errors: every entry point returns a bsa_status; invalid arguments are
 *     rejected before anything is enqueued.  No C++ exception crosses the ABI.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSA_API __attribute__((visibility("default")))

typedef int32_t bsa_status;
#define BSA_OK 0
#define BSA_ERR_INVALID_ARG (-1) /* null pointer, bad size, misaligned buffer   */
#define BSA_ERR_UNSUPPORTED (-2) /* D, block or nb outside the supported set     */
#define BSA_ERR_HIP (-3)         /* a HIP launch or runtime call failed          */
#define BSA_ERR_CAPACITY (-4)    /* workspace too small, or nnz beyond int32     */
#define BSA_ERR_PLAN_MISMATCH (-5) /* CSR rows do not match prior + budget plan */

/* Human-readable name of a status code (static string, never NULL). */
BSA_API const char* bsa_status_string(bsa_status s);

/* ABI version of this header (incremented on any signature change). */
#define BSA_ABI_VERSION 12

/* Largest number of item groups a work list may have (see bsa_work_plan_host). */
#define BSA_MAX_GROUPS 64
BSA_API int32_t bsa_abi_version(void);

/* ---------------------------------------------------------------- host plan */

/*
 * Blocks per query block for a target density (host, pure).
 * BSA-DiT §5.1 and the MC-Sparse summary (mean-pooled selection "at a given
 * attention density") fix a density, not a count; the count is
 *   K = 0                                   if density <= 0
 *   K = clamp(floor(density*nb + 0.5), 1, nb) otherwise.
 * Returns K, or -1 if nb < 1 or density is NaN.
 */
BSA_API int32_t bsa_budget_from_density(int32_t nb, double density);

/*
 * Data-independent CSR plan (host, synchronous).  BSA-DiT §2.3 (static prior
 * combined with dynamic selection) and §5.3 (a target count per query block):
 * row r keeps its prior blocks (plus the diagonal when force_diag != 0) and is
 * filled up to K_i blocks by score, so its length is max(|prior_i ∪ diag|, K_i)
 * whatever the data.
 *   prior_host    uint8 [nb*nb] (prior_per_head == 0) or [B*H*nb*nb] (!= 0),
 *                 nonzero = block kept; may be NULL (empty prior).
 *   budgets_host  int32 [nb] per-query-block K_i (shared by all heads), or NULL
 *                 to use K = bsa_budget_from_density(nb, density) for every row.
 *                 Values are clamped to [0, nb].
 *   row_ptr_out   int32 [B*H*nb + 1], written.
 *   nnz_out       total number of (row, column) entries, written (may be NULL).
 * Errors: INVALID_ARG for bad sizes or a NULL row_ptr_out; CAPACITY if nnz
 * would not fit in int32.
 */
BSA_API bsa_status bsa_mask_plan(int32_t B, int32_t H, int32_t nb, double density,
                                 const uint8_t* prior_host, int32_t prior_per_head,
                                 const int32_t* budgets_host, int32_t force_diag,
                                 int32_t* row_ptr_out, int64_t* nnz_out);

/*
 * Work list of bsa_forward (host, synchronous).  BSA-DiT §5.3: when query
 * blocks have very different active counts, one workgroup per query block
 * leaves some workgroups busy long after the others went idle; it suggests
 * sorting or merging the work, or per-block target counts.  Here every row
 * longer than max_tiles KV blocks is cut into near-equal chunks of at most
 * max_tiles blocks (max_tiles <= 0: rows are never cut); the chunks of a cut
 * row write fp32 partial results to the forward's workspace, and the forward
 * combines them once the last one is stored.
 * Groups and order: the items are split into n_groups groups (n_groups <= 1:
 * one group; at most BSA_MAX_GROUPS), meant for the accelerator dies (XCDs),
 * whose L2 caches are separate: workgroup i of the forward runs on die
 * i % n_groups and serves group i % n_groups.  Group g holds the heads
 * h = row / nb with h % n_groups == g.  Inside a group the chunks of cut rows
 * come first, then the whole rows; each class head by head, each head's
 * longest items first; ties keep ascending row, then chunk.
 * The forward's workgroups take the items of their group in that order (the
 * first two rounds statically, the rest from a per-group counter), so the
 * order is the dispatch order within a group.
 *   row_ptr   int32 [n_rows + 1] host copy of the CSR row pointer.
 *   nb        blocks per head (rows of one head are consecutive).
 *   work_out  int32 [capacity], written: n_items records {row, col_begin,
 *             col_end, slot}: the item covers col_idx[col_begin, col_end) of
 *             CSR row `row` (absolute positions; slot = -1: the item covers
 *             the whole row and writes O directly), grouped as above; then
 *             n_merges records {row, first_slot, n_chunks}; then the group
 *             table {G, s_0, s_1, ..., s_G}: G groups, group g being items
 *             [s_g, s_(g+1)) (s_0 = 0, s_G = n_items); then the slot map:
 *             n_slots ints, the merge record index of every partial slot.
 *             The list takes 4 n_items + 3 n_merges + G + 2 + n_slots ints.
 *   capacity  >= bsa_work_plan_ints(n_rows, nnz, max_tiles) int32 entries.
 *   n_items, n_merges, n_slots  written (n_slots = partial slots used).
 * Errors: INVALID_ARG for a NULL pointer, n_rows < 1, a decreasing row_ptr or
 * n_groups outside [0, BSA_MAX_GROUPS]; CAPACITY if capacity is too small.
 */
BSA_API int64_t bsa_work_plan_ints(int32_t n_rows, int64_t nnz, int32_t max_tiles);
BSA_API bsa_status bsa_work_plan_host(const int32_t* row_ptr, int32_t n_rows, int32_t nb,
                                      int32_t max_tiles, int32_t n_groups, int32_t* work_out,
                                      int64_t capacity, int32_t* n_items, int32_t* n_merges,
                                      int32_t* n_slots);

/*
 * Structural CSR check (host, synchronous): row_ptr[0] == 0, non-decreasing,
 * every column in [0, nb); strict == 1: also strictly ascending per row (which
 * implies distinct); strict == 2: distinct per row, in any order.
 * On failure returns INVALID_ARG and writes the first offending row to
 * *bad_row (if non-NULL); on success *bad_row = -1.
 */
BSA_API bsa_status bsa_validate_csr_host(const int32_t* row_ptr, const int32_t* col_idx,
                                         int32_t n_rows, int32_t nb, int32_t strict,
                                         int64_t* bad_row);

/* ------------------------------------------------------------- device calls */

/*
 * Bytes of device workspace bsa_build_mask needs: pooled Q and K (fp32
 * [B,H,nb,D] each), block scores (fp32 [B,H,nb,nb]) and a status word.
 */
BSA_API size_t bsa_build_mask_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t D,
                                              int32_t block);

/*
 * Mean-pool top-k block mask (device, async on `stream`).
 * MC-Sparse summary, section on mean-pooled block scoring: every query block
 * and KV block is represented by the mean of its (valid) tokens, every pair is
 * scored by the dot product of those means (fp32, no scale), and each query
 * block keeps its highest-scoring KV blocks; BSA-DiT §2.3: unioned with a
 * static prior; BSA-DiT §5.3: optional per-row target counts.
 *   q, k          bf16 [B,H,N,D] device.
 *   density       target density (used when budgets_dev is NULL).
 *   budgets_dev   int32 [nb] device, or NULL.
 *   prior_dev     uint8 [nb*nb] or [B*H*nb*nb] device, or NULL.
 *   force_diag    nonzero: block i is always kept in row i.
 *   row_ptr_dev   int32 [B*H*nb+1] device: MUST be the plan of bsa_mask_plan
 *                 for the same prior, budgets/density and force_diag.
 *   col_idx_dev   int32 [nnz] device, written: per row the prior (and diagonal)
 *                 plus the best max(0, K_i - |prior_i|) other blocks by
 *                 descending score (ties: lower column), in ascending order.
 *   workspace     device buffer of >= bsa_build_mask_workspace_bytes bytes.
 * Rows whose planned length disagrees with the prior and budget are left
 * unwritten and counted in the workspace status word; read it with
 * bsa_build_mask_status.  Errors: INVALID_ARG, UNSUPPORTED, CAPACITY, HIP.
 */
BSA_API bsa_status bsa_build_mask(const void* q, const void* k, int32_t B, int32_t H,
                                  int32_t N, int32_t D, int32_t block, double density,
                                  const int32_t* budgets_dev, const uint8_t* prior_dev,
                                  int32_t prior_per_head, int32_t force_diag,
                                  const int32_t* row_ptr_dev, int32_t* col_idx_dev,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Synchronously read the status word of the last bsa_build_mask that used
 * `workspace` (waits for `stream`): *mismatched_rows = number of rows whose
 * row_ptr length did not match the plan.  Returns PLAN_MISMATCH if nonzero.
 */
BSA_API bsa_status bsa_build_mask_status(const void* workspace, void* stream,
                                         int32_t* mismatched_rows);

/*
 * Longest-row-first work list built on the device (async), for a CSR whose
 * row lengths the host does not hold: the work_dev layout of
 * bsa_work_plan_host with one group and no row cut (n_items = n_rows,
 * n_merges = 0, every item {row, row_ptr[row], row_ptr[row + 1], -1}, then
 * the group table {1, 0, n_rows}), produced by a counting sort of the rows by
 * length, longest first (order among equal lengths unspecified; results do
 * not depend on it).
 *   row_ptr_dev int32 [n_rows+1]; work_dev int32 [4*n_rows + 3] written;
 *   max_len >= every row length (e.g. nb); at most 8191.
 */
BSA_API bsa_status bsa_schedule(const int32_t* row_ptr_dev, int32_t n_rows, int32_t max_len,
                                int32_t* work_dev, void* stream);

/*
 * Bytes of device workspace bsa_forward needs with a work list: 256 KiB of
 * item counters (one int32 per group, 4 KiB apart), then 2 n_slots int32 merge
 * counters (rounded up to 256 bytes), then n_slots partial results (fp32 O
 * [block x D] plus running max and sum per query row, per slot).
 */
BSA_API size_t bsa_forward_workspace_bytes(int32_t n_slots, int32_t D, int32_t block);

/*
 * Block-sparse attention forward (device, async on `stream`).
 * BSA-DiT §4.1: for every query block, only the KV blocks listed in its CSR
 * row are loaded and multiplied; BSA-DiT §4.3: the online softmax runs over
 * those blocks only and divides by their true total, so skipped blocks count
 * as score -inf.  Output:
 *   O[bi,h,a,:] = sum_c softmax_c(scale * q_a.k_c) v_c over active keys c,
 *   LSE[bi,h,a] = log sum_c exp(scale * q_a.k_c)       (natural log)
 * bf16 inputs, fp32 accumulation, O rounded to bf16 (nearest even).
 *   q, k, v     bf16 [B,H,N,D] device; o bf16 [B,H,N,D] device (written);
 *   lse         fp32 [B,H,N] device (written), or NULL to skip it.
 *   row_ptr_dev, col_idx_dev  the CSR (see conventions); entries outside
 *               [0, nb) contribute nothing, row bounds are clamped to [0, nnz].
 *   work_dev    device copy of a work list (bsa_work_plan_host or
 *               bsa_schedule) with n_items items and n_merges merges, or NULL
 *               for one item per row in natural order (n_items, n_merges
 *               ignored).  Every row must be covered exactly once; column
 *               ranges are clamped to [0, nnz].  Workgroups stay resident:
 *               without a list, workgroup w runs rows w, w + G, ... (G =
 *               workgroups launched); with one, workgroup w serves group
 *               w % n_groups, runs that group's items w / n_groups and
 *               w / n_groups + G_g (G_g = its group's workgroups) and then
 *               claims the group's remaining items in list order from a
 *               counter in the workspace.
 *   workspace   with a work list: >= bsa_forward_workspace_bytes(n_slots, D,
 *               block) bytes of device memory, 16-byte aligned, whose
 *               counters (item and merge counters) are zero before the first
 *               call; every call that completes leaves them zero again, so
 *               calls that use one workspace must be ordered on one stream.
 *               Without a list it may be NULL.  The partial results need no
 *               initialisation.
 *   scale       softmax scale; <= 0 means 1/sqrt(D).
 * A row with no active block yields O = 0 and LSE = -inf.
 * Errors: INVALID_ARG (also a work list without a workspace), UNSUPPORTED,
 * CAPACITY (workspace too small), HIP.
 */
BSA_API bsa_status bsa_forward(const void* q, const void* k, const void* v, int32_t B,
                               int32_t H, int32_t N, int32_t D, int32_t block,
                               const int32_t* row_ptr_dev, const int32_t* col_idx_dev,
                               const int32_t* work_dev, int32_t n_items, int32_t n_merges,
                               int32_t n_slots, float scale, void* o, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * bsa_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and arguments as bsa_forward, without the workspace.  With
 * a work list, the workspace bsa_forward would take (item and merge counters,
 * partial results of cut rows) lives in a static device array of
 * BSA_FORWARD_NOALLOC_MAX_BYTES that each GPU the library runs on holds until
 * the process ends; its device address is taken once per device, on the
 * first call with that device current.  Every call first clears the counters
 * (a small kernel on `stream`, no memset), then runs bsa_forward on it.
 * Calls on one GPU share the array: calls that may overlap (different
 * streams without ordering) race and must not be issued.  Without a work
 * list no workspace is used at all.  Nothing is allocated, no library routine
 * that allocates is called.
 * Errors: those of bsa_forward; CAPACITY when bsa_forward_workspace_bytes(
 * n_slots, D, block) exceeds BSA_FORWARD_NOALLOC_MAX_BYTES; HIP if the array's
 * address cannot be taken.
 */
#define BSA_FORWARD_NOALLOC_MAX_BYTES (16u << 20)
BSA_API bsa_status bsa_forward_noalloc(const void* q, const void* k, const void* v, int32_t B,
                                       int32_t H, int32_t N, int32_t D, int32_t block,
                                       const int32_t* row_ptr_dev, const int32_t* col_idx_dev,
                                       const int32_t* work_dev, int32_t n_items,
                                       int32_t n_merges, int32_t n_slots, float scale, void* o,
                                       float* lse, void* stream);

/*
 * Exact attention mass per block pair (device, async): the second pass of
 * exact block selection.  Page "Can sparse attention close the quality gap in
 * diffusion transformers": its oracle sections compare sparse attention, at
 * equal density, with oracles that keep the most mass of the exact dense
 * attention probabilities (the block oracle chooses KV blocks per query block);
 * its section on token-level selection notes that exact selection needs the
 * scores, which a FlashAttention pass does not expose, hence two passes.  The
 * first is bsa_forward with an all-ones CSR (its LSE); this is the second:
 *   mass[r, j] = sum over queries t of block i and keys c of block j (t, c < N)
 *                of exp(scale q_t.k_c - lse[bi,h,t]),   r = (bi*H + h)*nb + i.
 * With the dense LSE a mass row sums to the query count of its block.
 *   q, k       bf16 [B,H,N,D] device, 16-byte aligned.
 *   lse        fp32 [B,H,N] device: the dense natural-log LSE (queries with a
 *              non-finite LSE contribute nothing).
 *   scale      softmax scale; <= 0 means 1/sqrt(D) (must match the LSE's).
 *   mass_out   fp32 [B*H*nb, nb] device, written.
 * (block, D) as bsa_forward.  Errors: INVALID_ARG, UNSUPPORTED (shape, or a head
 * of 2^31 bytes or more), HIP.
 */
BSA_API bsa_status bsa_block_mass(const void* q, const void* k, const float* lse, int32_t B,
                                  int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                                  float* mass_out, void* stream);

/*
 * Block oracle at the density of a given CSR (device, async): for every row r,
 * the row_ptr[r+1] - row_ptr[r] KV blocks of largest mass[r, :] (ties to the
 * lower block index), written ascending to col_idx[row_ptr[r] ...].  Page "Can
 * sparse attention close the quality gap in diffusion transformers", oracle
 * sections: equal density, most retained mass.
 *   mass_dev     fp32 [n_rows, nb] device (bsa_block_mass), n_rows = B*H*nb.
 *   row_ptr_dev  int32 [n_rows + 1] device (the CSR whose density is matched).
 *   col_idx_dev  int32 [row_ptr[n_rows]] device, written.
 *   status_dev   int32 device word, set to the number of rows left unwritten
 *                (a row longer than nb or outside [0, nnz]); read it after the
 *                stream completes.
 * nb at most 1024.  Errors: INVALID_ARG, UNSUPPORTED (nb), HIP.
 */
BSA_API bsa_status bsa_select_by_mass(const float* mass_dev, int32_t n_rows, int32_t nb,
                                      const int32_t* row_ptr_dev, int32_t* col_idx_dev,
                                      int32_t* status_dev, void* stream);

/*
 * Retained mass of a CSR (device, async): out[r] = sum of mass[r, j] over the
 * blocks j listed in row r (columns outside [0, nb) ignored, row bounds clamped
 * to [0, nnz]); divided by the block's query count it is the mean attention
 * probability the row's queries keep.
 *   mass  fp32 [n_rows, nb] device; row_ptr int32 [n_rows + 1], col_idx int32
 *   [nnz] device; out fp32 [n_rows] device, written.
 * Errors: INVALID_ARG, HIP.
 */
BSA_API bsa_status bsa_csr_mass(const float* mass, int32_t n_rows, int32_t nb,
                                const int32_t* row_ptr, const int32_t* col_idx, float* out,
                                void* stream);

/*
 * Dense-sparse residual compensation (device, async).  Page "Can sparse
 * attention close the quality gap in diffusion transformers", section on
 * residual compensation: at an anchor step the residual between the dense and
 * the sparse attention outputs is recorded; at a reuse step (which reuses the
 * anchor's CSR, per the section on reusing exact selection) the cached residual
 * is added to the sparse output.
 *   bsa_residual:   r_out = o_dense - o_sparse
 *   bsa_compensate: o_out = o_sparse + r
 * All bf16 device arrays of n elements (e.g. [B,H,N,D]), 16-byte aligned; each
 * element is formed in fp32 from the two bf16 inputs and rounded once to bf16
 * (nearest even).  The output may alias an input.  Errors: INVALID_ARG, HIP.
 */
BSA_API bsa_status bsa_residual(const void* o_dense, const void* o_sparse, void* r_out, int64_t n,
                                void* stream);
BSA_API bsa_status bsa_compensate(const void* o_sparse, const void* r, void* o_out, int64_t n,
                                  void* stream);

/*
 * bsa_forward with the residual added in its epilogue (device, async): the
 * reuse step of the same section (sparse output plus the cached residual) in
 * one pass instead of bsa_forward followed by bsa_compensate.
 *   O[bi,h,a,:] = round_bf16(attention_fp32[bi,h,a,:] + r[bi,h,a,:]), the sum
 *   formed in fp32 from the unrounded attention output and r, rounded once to
 *   bf16 (nearest even); LSE is the attention's, as in bsa_forward.
 *   r   bf16 [B,H,N,D] device, 16-byte aligned (e.g. bsa_residual's output),
 *       not overlapping o.
 * Every other argument, the work list and workspace rules and the errors are
 * bsa_forward's; INVALID_ARG also for r NULL, misaligned or overlapping o.
 */
BSA_API bsa_status bsa_forward_compensated(const void* q, const void* k, const void* v,
                                           int32_t B, int32_t H, int32_t N, int32_t D,
                                           int32_t block, const int32_t* row_ptr_dev,
                                           const int32_t* col_idx_dev, const int32_t* work_dev,
                                           int32_t n_items, int32_t n_merges, int32_t n_slots,
                                           float scale, const void* r, void* o, float* lse,
                                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Token-level KV selection with tile-aligned query groups (device, async).  Page
 * "Can sparse attention close the quality gap in diffusion transformers",
 * section on token-level selection with tile-aligned query groups: KV tokens are
 * chosen one by one per query group and gathered by index; the queries of a head
 * form groups of C similar queries by the median-split version of
 * principal-direction divisive partitioning; exact selection needs the scores.
 *
 * bsa_query_groups: groups_out int32 [B,H,N/C,C] (token indices, each group
 *   ascending), from q bf16 [B,H,N,D].  Per head, a group of g*C queries (g > 1) is
 *   projected on its principal direction (8 power-iteration steps from
 *   u[d] = 1 + d/D, fp32) and cut into floor(g/2)*C and the rest, smallest
 *   projections first (ties to the lower token), recursively; groups are
 *   numbered depth first.  C in {64, 128}, N a multiple of C and at most 8192, D
 *   in {64, 128}, B*H at most 65535.  One level of the split tree per launch pair;
 *   the principal direction is iterated on the segment's scatter matrix
 *   sum (x - mu)(x - mu)^T (the same map as X_c^T X_c on the centred rows), which
 *   segments above 1024 tokens assemble from fp32 partials of 512-token slices.
 *   workspace: device, bsa_query_groups_workspace_bytes(B, H, N, D, C) bytes,
 *   16-byte aligned, no initial contents (the partials of one level at a time).
 * bsa_token_mass: mass_out fp32 [B,H,N/C,N]: for group g and token c, the sum over
 *   the group's queries t of exp(scale q_t.k_c - lse[t]) (with the dense LSE: the
 *   dense attention probability mass of token c for the group).  Queries with a
 *   non-finite LSE contribute nothing.
 * bsa_select_tokens: tokens_out int32 [n_rows, k]: per mass row, the k tokens of
 *   largest mass (ties to the lower token), ascending.  N at most 8192, 0 <= k <= N.
 * Errors: INVALID_ARG, UNSUPPORTED (sizes above), HIP.
 */
BSA_API size_t bsa_query_groups_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t D,
                                                int32_t C);
BSA_API bsa_status bsa_query_groups(const void* q, int32_t B, int32_t H, int32_t N, int32_t D,
                                    int32_t C, int32_t* groups_out, void* workspace,
                                    size_t workspace_bytes, void* stream);
BSA_API bsa_status bsa_token_mass(const void* q, const void* k, const float* lse,
                                  const int32_t* groups, int32_t B, int32_t H, int32_t N,
                                  int32_t D, int32_t C, float scale, float* mass_out,
                                  void* stream);
BSA_API bsa_status bsa_select_tokens(const float* mass, int32_t n_rows, int32_t N, int32_t k,
                                     int32_t* tokens_out, void* stream);

/*
 * Gathered attention over selected tokens (device, async).  Same page and section:
 * the selected KV tokens of a query group are gathered by index, not repacked into
 * blocks, and the group's queries attend to exactly those tokens.
 *
 * q, k, v: bf16 [B,H,N,D], D = 64 or 128, 16-byte aligned.  groups: int32 [B,H,G,64], the
 * token positions of each group's 64 queries (as bsa_query_groups writes them with
 * C = 64).  tokens: int32 [B,H,G,T], the KV tokens of each group (as
 * bsa_select_tokens writes them); a list must not repeat a token (a repeat counts
 * twice), its order is free.  Entries outside [0, N) are skipped in both.  For
 * every query t of group g: o[t] = softmax_j(scale q_t.k_j) v_j over j in tokens[g]
 * (fp32 accumulation, bf16 result) and lse[t] = log sum_j exp(scale q_t.k_j),
 * natural log, fp32 [B,H,N]; a group with no valid token writes o = 0 and
 * lse = -inf.  Rows of o and lse that no group names are not written.  scale <= 0
 * selects 1/sqrt(D); lse may be NULL.
 * Errors: INVALID_ARG (null or misaligned pointer, non-positive sizes, NaN scale),
 * UNSUPPORTED (D not 64 or 128, N*D*2 >= 2^31), HIP.
 */
BSA_API bsa_status bsa_gather_forward(const void* q, const void* k, const void* v, int32_t B,
                                      int32_t H, int32_t N, int32_t D, const int32_t* groups,
                                      int32_t G, const int32_t* tokens, int32_t T, float scale,
                                      void* o, float* lse, void* stream);

/*
 * Backward of the CSR forward (device, async).  BSA-DiT §2.3 and §5.2 train with
 * the block mask; the gradient is that of the forward's definition (§4.1, §4.3:
 * listed blocks visited, skipped blocks as -inf scores) for an incoming dO of O:
 *   P = exp(scale q.k - LSE) on listed keys < N (0 elsewhere), dV = P^T dO,
 *   dP = dO V^T, delta_t = sum_d dO[t,d] O[t,d], dS = P (dP - delta),
 *   dQ = scale dS K, dK = scale dS^T Q.
 * q, k, v, o, d_o: bf16 [B,H,N,D]; lse fp32 [B,H,N]: O and LSE of bsa_forward over
 * the same CSR and scale.  dq, dk, dv: bf16 [B,H,N,D], every row written (keys that
 * no row lists and queries of empty rows get 0); they must not alias the inputs.
 * row_ptr, col_idx: the forward's CSR (device); columns of a row must be distinct
 * (a repeat counts once here but twice in the forward); columns outside [0, nb)
 * are ignored.  nnz: an upper bound of row_ptr[B*H*nb] (sizes the workspace).
 * scale <= 0 selects 1/sqrt(D).  Accumulation in fp32, P and dS rounded to bf16 as
 * MFMA operands; no atomics on the gradients, so results are deterministic.
 * workspace: device, bsa_backward_workspace_bytes(B, H, N, D, block, nnz) bytes, 16-byte
 * aligned; it holds (LSE log2 e, delta) per query row, the transposed CSR, the split
 * of key columns and CSR rows longer than the chunk length (twice the mean row
 * length, at least 16) into chunks, the work lists of the two gradient kernels (one
 * per die, 8, when B*H >= 8, else one; 16-byte records), at D = 128 the bf16 dS
 * tile of every listed block pair (nnz x 8 KiB, written by the dK/dV pass and
 * read by the dQ pass instead of recomputing it), and the chunks' fp32 partial
 * gradients (bounded by 2 nnz / chunk + 1 slots of 768 D bytes); it needs no
 * initial contents.  Calls that share a workspace must not overlap.  With
 * block = 128 the CSR is first refined to the 64-block CSR of the same mask (query
 * block i is query blocks 2i, 2i + 1 and key block j key blocks 2j, 2j + 1; at most
 * 4 nnz entries, held in the workspace), and the rest works on that.
 * Supported: D = 64 or 128, block = 64 or 128, ceil(N / 64) <= 1024.
 * Errors: INVALID_ARG (null or misaligned pointer, bad size, NaN scale),
 * UNSUPPORTED (D, block, nb), CAPACITY (workspace too small), HIP.
 */
BSA_API size_t bsa_backward_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t D,
                                            int32_t block, int64_t nnz);
BSA_API bsa_status bsa_backward(const void* q, const void* k, const void* v, const void* o,
                                const void* d_o, const float* lse, int32_t B, int32_t H,
                                int32_t N, int32_t D, int32_t block, const int32_t* row_ptr,
                                const int32_t* col_idx, int64_t nnz, float scale, void* dq,
                                void* dk, void* dv, void* workspace, size_t workspace_bytes,
                                void* stream);

#ifdef __cplusplus
}
#endif
#endif /* BSA_H */
