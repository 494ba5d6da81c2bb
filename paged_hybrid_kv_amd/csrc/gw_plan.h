// Split plan shared by host (grid and workspace sizing) and device (what each
// workgroup does).  A row's plan depends only on the number of pages its own
// attended range covers, never on the other rows of the call, their order or
// where pages sit, so every row's result is the same whatever batch it is in.
#pragma once

#include <hip/hip_runtime.h>

namespace gw {

// Local family: ranges up to the window (65 pages at window 1024).  A
// workgroup has 8 waves at query-group size 1 or 2 and takes splits of at
// least 33 pages: a full window is 2 splits, so 16 rows x 8 KV heads fill
// the GPU with 256 workgroups of 8 waves in one round.  At group size 4 the
// registers of 8 waves do not suffice: 4 waves, splits of at least 17 pages
// (4 per full window, 512 workgroups).
constexpr int kLocalMaxSplits = 16;
__host__ __device__ constexpr int local_waves(int group) { return group >= 4 ? 4 : 8; }
__host__ __device__ constexpr int local_min_pages_per_split(int group) { return group >= 4 ? 17 : 33; }
// Most consecutive splits one local decode workgroup takes: a wave keeps
// one softmax state per split, and the bf16 pages of group sizes 1 and 2
// leave no registers for a second (the 4-wave workgroups of group size 4
// have twice the registers per wave).
__host__ __device__ constexpr int local_max_splits_per_wg(int group, bool fp8) {
  return fp8 ? (group >= 4 ? 4 : 2) : (group >= 4 ? 2 : 1);
}

// Global family: splits of at least 20 pages (320 tokens), at most 64 per
// row unless that would put more than 256 pages in one split: 16 rows of
// 2K..8K tokens make about 250 workgroups, one per CU in a single round; a
// row takes 64 splits from 20K tokens on, and more from 256K tokens on.
constexpr int kGlobalMinPagesPerSplit = 20;
constexpr int kGlobalMaxSplits = 64;
constexpr int kGlobalMaxPagesPerSplit = 256;

__host__ __device__ inline int cdiv_i(int a, int b) { return (a + b - 1) / b; }

__host__ __device__ inline int local_nsplit(int n_pages, int group) {
  int k = cdiv_i(n_pages, local_min_pages_per_split(group));
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

// Balanced split of n units into k parts: part i is [split_lo(n, k, i),
// split_lo(n, k, i + 1)), i.e. floor(n i / k).  Written as
// (n / k) i + ((n % k) i) / k, which is the same integer (n = (n / k) k +
// n % k, and (n / k) i is whole) but never forms the product n i: the first
// term is at most n and the second's product is below k^2, so every value
// stays in 32 bits for any n < 2^31 and k <= kMaxSplitsAny.  (n i itself
// would pass 2^32 for the longest rows served, 2^20 pages split 4096 ways.)
constexpr int kMaxSplitsAny = 46340;   // k^2 < 2^31
__host__ __device__ inline int split_lo(int n, int k, int i) {
  const int q = n / k, r = n - q * k;
  return q * i + (r * i) / k;
}

// Prompt rows (sequences with more than one query row in a call).  A local
// prompt-row workgroup takes kLocalPrefillVectors query vectors (a row and
// one q head of its group): 128 / G consecutive rows of one (sequence, KV
// head).  A global one takes 8 / HB rows (HB = q heads / 16).  Upper bound
// on a call's (prompt sequence, row block) items: every sequence's rows in
// blocks of `rows`, at most (rows of the call + sequences (rows - 1)) / rows
// and at most sequences x ceil(max_q_len / rows).
constexpr int kLocalPrefillVectors = 128;
__host__ __device__ constexpr int local_prefill_rows(int group) { return kLocalPrefillVectors / group; }
__host__ __device__ constexpr int global_prefill_rows(int num_q_heads) { return num_q_heads == 32 ? 4 : 8; }
inline long long prefill_items(long long num_rows, long long num_seqs, long long max_q_len, long long rows) {
  const long long by_rows = (num_rows + num_seqs * (rows - 1)) / rows;
  const long long by_len = num_seqs * ((max_q_len + rows - 1) / rows);
  return by_rows < by_len ? by_rows : by_len;
}

// Units of 256 threads of the global cross-split reduce per decode
// sequence, in its sequential schedule: four 16-head x 16-dim output
// fragments each (32 fragments per block of 16 q heads).
__host__ __device__ constexpr int reduce_groups(int num_q_heads) { return num_q_heads / 16 * 32 / 4; }

// Page items of the prompt rows' append in an attention call: a sequence
// of q rows touches at most (q + 14) / 16 + 1 pages, so the call at most
// (rows + 30 sequences) / 16 (and at most sequences * pages of max_q_len).
// A local item covers kRowsAppendHeads KV heads of its page.
constexpr int kRowsAppendHeads = 2;
inline long long rows_append_items(long long num_rows, long long num_seqs, long long max_q_len) {
  const long long by_rows = (num_rows + 30 * num_seqs) / 16;
  const long long by_len = num_seqs * ((max_q_len + 14) / 16 + 1);
  return by_rows < by_len ? by_rows : by_len;
}

// Pages touched by the window of a query at position p: [p_lo/16, p/16].
__host__ __device__ inline int local_range_pages(int p, int window) {
  int lo = p - window + 1;
  lo = lo < 0 ? 0 : lo;
  return p / 16 - lo / 16 + 1;
}

// The local range [lo, p] of a decode row at position p, walked as
// "virtual pages".  The range touches pages pg0 = lo/16 .. pgl = p/16; when
// the first page's slots in use [lo%16, 15] and the last page's [0, p%16]
// are disjoint (a full window that does not start on a page boundary), the
// two are walked as one page, slot t taken from the first page when
// t >= lo%16 and from the last page otherwise.  A full 1024-token window is
// then 64 pages of work rather than 65 (the same bytes: the two edge pages
// together hold exactly 16 slots of the window).  Virtual page 0 is that
// merged page (wrap) or page pg0; virtual page v >= 1 is page pg0 + v.
struct LocalWindow {
  int lo, pg0, pgl;
  int nv;       // virtual pages
  int b;        // wrap: first slot read from page pg0 (the rest from pgl); else 0
  bool wrap;
};

__host__ __device__ inline LocalWindow local_window(int p, int window) {
  LocalWindow r;
  r.lo = p - window + 1 < 0 ? 0 : p - window + 1;
  r.pg0 = r.lo / 16;
  r.pgl = p / 16;
  const int npg = r.pgl - r.pg0 + 1;
  r.wrap = npg >= 2 && (p % 16) < (r.lo % 16);
  r.nv = r.wrap ? npg - 1 : npg;
  r.b = r.wrap ? r.lo % 16 : 0;
  return r;
}

// Upper bound on pages of any local decode range for sequences <= max_len
// (it also bounds the virtual page count).
inline int local_max_range_pages(int max_len, int window) {
  int w = window < max_len ? window : max_len;
  // a w-token range starting mid-page spans at most cdiv(w - 1, 16) + 1 pages
  return cdiv_i(w - 1, 16) + 1;
}

}  // namespace gw
