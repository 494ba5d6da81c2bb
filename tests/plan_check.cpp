// Exhaustive host check of the split plans in gw_plan.h (built and run by
// tests/test_plan.py).  For every page count n up to 2^20 (the pages of the
// longest row the entry points accept, 2^24 tokens) and every split count
// the plans choose:
//   - split_lo(n, k, i) equals floor(n i / k) computed in 64 bits,
//   - the parts tile [0, n) in order with no empty part,
//   - a global part holds at most kGlobalMaxPagesPerSplit pages, and the
//     global plan uses at most kGlobalMaxSplits splits unless that bound
//     forces more; a local plan uses at most kLocalMaxSplits splits.
// Prints "ok <checks>" and exits 0, or prints the first failure and exits 1.
#include <cstdint>
#include <cstdio>

#include "gw_plan.h"

using namespace gw;

static long long g_checks = 0;

static bool partition(int n, int k, int max_part, const char* what) {
  if (k < 1 || k > kMaxSplitsAny) {
    std::printf("%s: n=%d gives k=%d\n", what, n, k);
    return false;
  }
  int prev = 0;
  for (int i = 0; i <= k; ++i) {
    const int lo = split_lo(n, k, i);
    const long long ref = (long long)n * i / k;
    ++g_checks;
    if (lo != ref) {
      std::printf("%s: split_lo(%d, %d, %d) = %d, floor(n i / k) = %lld\n", what, n, k, i, lo, ref);
      return false;
    }
    if (i == 0 && lo != 0) return std::printf("%s: first part starts at %d\n", what, lo), false;
    if (i > 0) {
      const int len = lo - prev;
      if (len < 1 || len > max_part) {
        std::printf("%s: n=%d k=%d part %d holds %d pages (1 .. %d)\n", what, n, k, i - 1, len, max_part);
        return false;
      }
    }
    prev = lo;
  }
  if (prev != n) return std::printf("%s: n=%d parts end at %d\n", what, n, prev), false;
  return true;
}

int main() {
  const int kMaxPages = 1 << 20;
  for (int n = 1; n <= kMaxPages; ++n) {
    const int k = global_nsplit(n);
    const int forced = cdiv_i(n, kGlobalMaxPagesPerSplit);
    if (k > kGlobalMaxSplits && k != forced) {
      std::printf("global: n=%d k=%d above %d without need\n", n, k, kGlobalMaxSplits);
      return 1;
    }
    if (k > n) return std::printf("global: n=%d k=%d > n\n", n, k), 1;
    if (!partition(n, k, kGlobalMaxPagesPerSplit, "global")) return 1;
  }
  for (int group : {1, 2, 4}) {
    for (int n = 1; n <= kMaxPages; ++n) {
      const int k = local_nsplit(n, group);
      if (k > kLocalMaxSplits || k > n) return std::printf("local G=%d: n=%d k=%d\n", group, n, k), 1;
      if (!partition(n, k, n, "local")) return 1;
    }
  }
  // the local window's virtual pages never exceed the bound used to size
  // the workspace, for every position of a few windows
  for (int window : {1, 7, 15, 16, 17, 33, 1000, 1024, 1025, 4096}) {
    for (int p = 0; p < 3 * window + 64; ++p) {
      const LocalWindow w = local_window(p, window);
      const int bound = local_max_range_pages(p + 1, window);
      ++g_checks;
      if (w.nv < 1 || w.nv > bound) {
        std::printf("local window %d at p=%d: %d virtual pages, bound %d\n", window, p, w.nv, bound);
        return 1;
      }
    }
  }
  std::printf("ok %lld\n", g_checks);
  return 0;
}
