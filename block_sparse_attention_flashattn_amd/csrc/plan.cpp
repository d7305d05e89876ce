// Host-side planning: density -> count, CSR row lengths, launch order, CSR check.
//
// BSA-DiT §5.3 (last paragraph): static structure is prepared ahead of time and
// nothing data-dependent is built on the CPU.  Everything here depends only on
// sizes, the static prior and the budgets, never on Q/K/V, so it runs once per
// shape and prior and its results can be cached across calls.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "bsa.h"

extern "C" BSA_API const char* bsa_status_string(bsa_status s) {
  switch (s) {
    case BSA_OK: return "BSA_OK";
    case BSA_ERR_INVALID_ARG: return "BSA_ERR_INVALID_ARG";
    case BSA_ERR_UNSUPPORTED: return "BSA_ERR_UNSUPPORTED";
    case BSA_ERR_HIP: return "BSA_ERR_HIP";
    case BSA_ERR_CAPACITY: return "BSA_ERR_CAPACITY";
    case BSA_ERR_PLAN_MISMATCH: return "BSA_ERR_PLAN_MISMATCH";
    default: return "BSA_ERR_UNKNOWN";
  }
}

extern "C" BSA_API int32_t bsa_abi_version(void) { return BSA_ABI_VERSION; }

extern "C" BSA_API int32_t bsa_budget_from_density(int32_t nb, double density) {
  if (nb < 1 || density != density) return -1;
  if (density <= 0.0) return 0;
  double k = floor(density * static_cast<double>(nb) + 0.5);
  if (k < 1.0) k = 1.0;
  if (k > static_cast<double>(nb)) k = static_cast<double>(nb);
  return static_cast<int32_t>(k);
}

extern "C" BSA_API bsa_status bsa_mask_plan(int32_t B, int32_t H, int32_t nb, double density,
                                            const uint8_t* prior_host, int32_t prior_per_head,
                                            const int32_t* budgets_host, int32_t force_diag,
                                            int32_t* row_ptr_out, int64_t* nnz_out) {
  if (B < 1 || H < 1 || nb < 1 || !row_ptr_out || density != density) return BSA_ERR_INVALID_ARG;
  const int32_t kd = bsa_budget_from_density(nb, density);
  const int64_t n_rows = int64_t(B) * H * nb;
  if (n_rows > INT32_MAX - 1) return BSA_ERR_CAPACITY;
  int64_t acc = 0;
  row_ptr_out[0] = 0;
  for (int64_t bh = 0; bh < int64_t(B) * H; ++bh) {
    for (int32_t i = 0; i < nb; ++i) {
      int64_t sel = 0;
      if (prior_host) {
        const uint8_t* row =
            prior_host + (prior_per_head ? bh * nb * nb : int64_t(0)) + int64_t(i) * nb;
        for (int32_t j = 0; j < nb; ++j) sel += row[j] ? 1 : 0;
        if (force_diag && !row[i]) ++sel;
      } else if (force_diag) {
        sel = 1;
      }
      int64_t ki = kd;
      if (budgets_host) {
        ki = budgets_host[i];
        if (ki < 0) ki = 0;
        if (ki > nb) ki = nb;
      }
      acc += sel > ki ? sel : ki;
      if (acc > INT32_MAX) return BSA_ERR_CAPACITY;
      row_ptr_out[bh * nb + i + 1] = static_cast<int32_t>(acc);
    }
  }
  if (nnz_out) *nnz_out = acc;
  return BSA_OK;
}

extern "C" BSA_API int64_t bsa_work_plan_ints(int32_t n_rows, int64_t nnz, int32_t max_tiles) {
  if (n_rows < 1 || nnz < 0) return -1;
  // Cutting a row of length L > T into ceil(L/T) chunks adds at most L/T items
  // and uses at most 2L/T partial slots (one map entry each); the group table
  // takes at most 2 + BSA_MAX_GROUPS ints.
  const int64_t extra = max_tiles > 0 ? nnz / max_tiles : 0;
  const int64_t slots = max_tiles > 0 ? 2 * nnz / max_tiles : 0;
  return 4 * (int64_t(n_rows) + extra) + 3 * int64_t(n_rows) + 2 + BSA_MAX_GROUPS + slots;
}

extern "C" BSA_API bsa_status bsa_work_plan_host(const int32_t* row_ptr, int32_t n_rows,
                                                 int32_t nb, int32_t max_tiles, int32_t n_groups,
                                                 int32_t* work_out, int64_t capacity,
                                                 int32_t* n_items, int32_t* n_merges,
                                                 int32_t* n_slots) {
  if (!row_ptr || !work_out || !n_items || !n_merges || !n_slots || n_rows < 1)
    return BSA_ERR_INVALID_ARG;
  if (n_groups < 0 || n_groups > BSA_MAX_GROUPS) return BSA_ERR_INVALID_ARG;
  struct Item { int32_t row, b, e, slot; };
  std::vector<Item> items;
  std::vector<int32_t> merges;
  items.reserve(size_t(n_rows));
  int32_t slots = 0;
  for (int32_t r = 0; r < n_rows; ++r) {
    const int32_t len = row_ptr[r + 1] - row_ptr[r];
    if (len < 0) return BSA_ERR_INVALID_ARG;
    if (max_tiles > 0 && len > max_tiles) {
      // Near-equal chunks: the first (len % n) chunks carry one extra tile.
      const int32_t n = (len + max_tiles - 1) / max_tiles;
      const int32_t base = len / n, rem = len % n;
      merges.push_back(r);
      merges.push_back(slots);
      merges.push_back(n);
      int32_t b = 0;
      for (int32_t c = 0; c < n; ++c) {
        const int32_t e = b + base + (c < rem ? 1 : 0);
        items.push_back({r, b, e, slots + c});
        b = e;
      }
      slots += n;
    } else {
      items.push_back({r, 0, len, -1});
    }
  }
  // Groups: head h = row / nb goes to group h % n_groups (the die whose
  // workgroups serve that group; workgroup i runs on die i % n_groups).  Inside
  // a group the chunks of cut rows (the largest items) come first, then the
  // whole rows; each class head by head, a head's longest items first.  Heads
  // in order keep the die's L2 on the K/V of about one head at a time (ordering
  // rows by length across heads instead ran as fast but doubled the L2 misses);
  // big items first leave small ones for the end, where early finishers claim
  // them.
  const int32_t ng = (nb > 0 && n_groups > 1) ? n_groups : 1;
  std::vector<std::vector<Item>> g(static_cast<size_t>(ng));
  for (const Item& it : items) g[ng > 1 ? size_t((it.row / nb) % ng) : 0].push_back(it);
  for (auto& x : g)
    std::stable_sort(x.begin(), x.end(), [nb](const Item& a, const Item& b) {
      const bool ca = a.slot >= 0, cb = b.slot >= 0;
      if (ca != cb) return ca;
      const int32_t ha = nb > 0 ? a.row / nb : 0, hb = nb > 0 ? b.row / nb : 0;
      return ha != hb ? ha < hb : a.e - a.b > b.e - b.b;
    });
  const int64_t need = 4 * int64_t(items.size()) + int64_t(merges.size()) + 2 + ng + slots;
  if (need > capacity) return BSA_ERR_CAPACITY;
  size_t k = 0;
  std::vector<int32_t> table;
  table.push_back(ng);
  for (const auto& x : g) {
    table.push_back(static_cast<int32_t>(k));
    for (const Item& it : x) {
      // Column positions are absolute indices into col_idx.
      const int32_t base = row_ptr[it.row];
      work_out[4 * k + 0] = it.row;
      work_out[4 * k + 1] = base + it.b;
      work_out[4 * k + 2] = base + it.e;
      work_out[4 * k + 3] = it.slot;
      ++k;
    }
  }
  table.push_back(static_cast<int32_t>(k));
  memcpy(work_out + 4 * k, merges.data(), merges.size() * sizeof(int32_t));
  memcpy(work_out + 4 * k + merges.size(), table.data(), table.size() * sizeof(int32_t));
  // Slot map: the merge record of every partial slot.
  int32_t* slot_merge = work_out + 4 * k + merges.size() + table.size();
  for (size_t m = 0; m < merges.size() / 3; ++m)
    for (int32_t c = 0; c < merges[3 * m + 2]; ++c) slot_merge[merges[3 * m + 1] + c] = int32_t(m);
  *n_items = static_cast<int32_t>(k);
  *n_merges = static_cast<int32_t>(merges.size() / 3);
  *n_slots = slots;
  return BSA_OK;
}

extern "C" BSA_API bsa_status bsa_validate_csr_host(const int32_t* row_ptr,
                                                    const int32_t* col_idx, int32_t n_rows,
                                                    int32_t nb, int32_t strict,
                                                    int64_t* bad_row) {
  if (bad_row) *bad_row = -1;
  if (!row_ptr || n_rows < 1 || nb < 1) return BSA_ERR_INVALID_ARG;
  if (row_ptr[0] != 0) {
    if (bad_row) *bad_row = 0;
    return BSA_ERR_INVALID_ARG;
  }
  // strict == 2: a column already seen in this row carries the row's stamp.
  std::vector<int32_t> seen(strict == 2 ? size_t(nb) : 0, -1);
  for (int32_t r = 0; r < n_rows; ++r) {
    const int32_t a = row_ptr[r], b = row_ptr[r + 1];
    bool ok = b >= a && (b == a || col_idx != nullptr);
    for (int32_t t = a; ok && t < b; ++t) {
      const int32_t c = col_idx[t];
      if (c < 0 || c >= nb) {
        ok = false;
      } else if (strict == 2) {
        if (seen[size_t(c)] == r) ok = false;
        seen[size_t(c)] = r;
      } else if (strict && t > a && col_idx[t - 1] >= c) {
        ok = false;
      }
    }
    if (!ok) {
      if (bad_row) *bad_row = r;
      return BSA_ERR_INVALID_ARG;
    }
  }
  return BSA_OK;
}
