// Longest-row-first launch order built on the device.
//
// BSA-DiT §5.3: when query blocks have very different active counts, a plain
// one-workgroup-per-query-block launch leaves some workgroups busy while others
// idle; it suggests sorting the work.  The forward launches CSR rows in the
// order written here: a counting sort of the rows by length, longest first,
// so the long rows start while the short ones fill in behind them.
//
// One workgroup of 1024 threads: LDS histogram by (max_len - length), a
// two-level exclusive scan, then an atomic scatter of {row, begin, end, -1}
// work items (no row is cut), then a one-group table.  Rows of equal length
// come out in an unspecified order; the forward's results do not depend on it.
#include "common.h"

namespace bsa {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kSchedMaxLen = 8191;

__global__ __launch_bounds__(kSchedThreads) void sched_kernel(const int32_t* __restrict__ row_ptr,
                                                              int32_t n_rows, int32_t max_len,
                                                              int32_t* __restrict__ work) {
  __shared__ int32_t bins[kSchedMaxLen + 1];
  __shared__ int32_t part[kSchedThreads];
  const int tid = threadIdx.x;
  const int nbins = max_len + 1;
  for (int b = tid; b < nbins; b += kSchedThreads) bins[b] = 0;
  __syncthreads();
  for (int r = tid; r < n_rows; r += kSchedThreads) {
    const int len = min(max(row_ptr[r + 1] - row_ptr[r], 0), max_len);
    atomicAdd(&bins[max_len - len], 1);
  }
  __syncthreads();
  // Exclusive scan: each thread owns a contiguous run of bins.
  const int per = (nbins + kSchedThreads - 1) / kSchedThreads;
  const int b0 = min(tid * per, nbins);
  const int b1 = min(b0 + per, nbins);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += bins[b];
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {
    const int add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int run = part[tid] - local;
  for (int b = b0; b < b1; ++b) {
    const int c = bins[b];
    bins[b] = run;
    run += c;
  }
  __syncthreads();
  for (int r = tid; r < n_rows; r += kSchedThreads) {
    const int b = row_ptr[r];
    const int full = max(row_ptr[r + 1] - b, 0);
    const int pos = atomicAdd(&bins[max_len - min(full, max_len)], 1);
    *reinterpret_cast<int4*>(work + 4 * size_t(pos)) = make_int4(r, b, b + full, -1);
  }
  if (tid == 0) {
    // Group table: one group holding every item.
    work[4 * size_t(n_rows) + 0] = 1;
    work[4 * size_t(n_rows) + 1] = 0;
    work[4 * size_t(n_rows) + 2] = n_rows;
  }
}

}  // namespace
}  // namespace bsa

extern "C" BSA_API bsa_status bsa_schedule(const int32_t* row_ptr_dev, int32_t n_rows,
                                           int32_t max_len, int32_t* work_dev, void* stream) {
  if (!row_ptr_dev || !work_dev || n_rows < 1 || max_len < 0) return BSA_ERR_INVALID_ARG;
  if (max_len > bsa::kSchedMaxLen) return BSA_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(work_dev) & 15u) return BSA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(bsa::sched_kernel, dim3(1), dim3(bsa::kSchedThreads), 0,
                     static_cast<hipStream_t>(stream), row_ptr_dev, n_rows, max_len, work_dev);
  BSA_HIP_CHECK_LAUNCH();
  return BSA_OK;
}
