// Split plan shared by host (grid and workspace sizing) and device (what each
// workgroup does).  A row's plan depends only on the number of pages its own
// attended range covers, never on the other rows of the call, their order or
// where pages sit, so every row's result is the same whatever batch it is in.
#pragma once

#include <hip/hip_runtime.h>

namespace gw {

// Local family: ranges up to the window (65 pages at window 1024) cut into
// splits of at least 17 pages: 4 splits of 16-17 pages for a full window,
// so 16 rows x 8 KV heads fill the GPU with 512 workgroups in one round.
constexpr int kLocalMinPagesPerSplit = 17;
constexpr int kLocalMaxSplits = 16;

// Global family: splits of at least 20 pages (320 tokens), at most 64 per
// row unless that would put more than 256 pages in one split: 16 rows of
// 2K..8K tokens make about 250 workgroups, one per CU in a single round; a
// row takes 64 splits from 20K tokens on, and more from 256K tokens on.
constexpr int kGlobalMinPagesPerSplit = 20;
constexpr int kGlobalMaxSplits = 64;
constexpr int kGlobalMaxPagesPerSplit = 256;

__host__ __device__ inline int cdiv_i(int a, int b) { return (a + b - 1) / b; }

__host__ __device__ inline int local_nsplit(int n_pages) {
  int k = cdiv_i(n_pages, kLocalMinPagesPerSplit);
  k = k < 1 ? 1 : k;
  return k > kLocalMaxSplits ? kLocalMaxSplits : k;
}

__host__ __device__ inline int global_nsplit(int n_pages) {
  int k = cdiv_i(n_pages, kGlobalMinPagesPerSplit);
  k = k < 1 ? 1 : k;
  k = k > kGlobalMaxSplits ? kGlobalMaxSplits : k;
  const int k_min = cdiv_i(n_pages, kGlobalMaxPagesPerSplit);
  return k < k_min ? k_min : k;
}

// Pages touched by the window of a query at position p: [p_lo/16, p/16].
__host__ __device__ inline int local_range_pages(int p, int window) {
  int lo = p - window + 1;
  lo = lo < 0 ? 0 : lo;
  return p / 16 - lo / 16 + 1;
}

// Upper bound on pages of any local decode range for sequences <= max_len.
inline int local_max_range_pages(int max_len, int window) {
  int w = window < max_len ? window : max_len;
  // a w-token range starting mid-page spans at most cdiv(w - 1, 16) + 1 pages
  return cdiv_i(w - 1, 16) + 1;
}

}  // namespace gw
