// Host page allocator of the two families and the page-copy launch
// (gw_alloc.hip), used by the C ABI (gw_api.hip).
#pragma once

#include <vector>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gw {

struct Allocator {
  struct Seq {
    bool used;
    int total, rows, len, first_query, res_l, res_g;
    std::vector<int> lpt, gpt;   // logical page -> physical page, -1 if none
  };
  int slots, max_context, window, local_pages, global_pages;
  int reserved_l = 0, reserved_g = 0;
  std::vector<int> free_local, free_global;   // descending: lowest id on top
  std::vector<Seq> seq;

  Allocator(int slots, int max_context, int window, int local_pages, int global_pages);
  int local_reserve(int total, int rows) const;
  int active() const;
  int admit(int total, int rows, int* slot);
  int extend(int slot, int new_len, int first_query);
  void release(int slot);
  static int take(std::vector<int>& fl);
  static void give(std::vector<int>& fl, int id);
};

hipError_t launch_copy_pages(uint8_t* dst, const uint8_t* src, const int32_t* dst_pages, const int32_t* src_pages,
                             int n, int64_t page_bytes, int64_t dst_num_pages, int64_t src_num_pages,
                             hipStream_t stream);

}  // namespace gw
