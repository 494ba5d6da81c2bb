// Host page allocator for the two families, and the page-copy kernel.
//
// Policy (pegainfer "Gemma 4" page, Scheduling): each family has its own
// paged pool and budget, 16-token pages in both; a request is admitted when
// a decode slot is free and both pools can hold it, its total length
// (prompt + max_tokens) checked against the ceiling at admission; otherwise
// it waits, and is refused only when nothing else runs (no pages can free
// up).  Local layers free the front of the window: pages wholly before the
// window of the earliest row still to be queried.  Global layers free
// nothing until the request ends, so a request's global footprint is its
// whole length.
//
// Admission reserves each request's worst case in each family: global, all
// ceil(total / 16) pages; local, the pages that one step's rows and their
// windows can span: rows + W - 1 tokens, at any offset in a page, touch at
// most (rows + W + 13) / 16 + 1 pages, and never more than ceil(total / 16).
// `rows` is the most rows one step queries.  Pages are then taken from the free lists as
// the sequence grows and can never run out; freed local pages go back at
// once.  Physical ids are handed out lowest first (free lists kept sorted
// as stacks of descending ids), so an allocator's state depends only on the
// sequence of calls.
//
// (Conversation prefix cache, same page: finished prompt states are kept
// in pages of their own and copied back on a hit -- gw_copy_pages.)

#include <algorithm>
#include <vector>

#include "gw_alloc.h"
#include "gw_device.h"

namespace gw {

int Allocator::local_reserve(int total, int rows) const {
  const int all = (total + kPage - 1) / kPage;
  const int span = (rows + window + 13) / kPage + 1;
  return std::min(all, span);
}

int Allocator::take(std::vector<int>& fl) {
  if (fl.empty()) return -1;
  const int id = fl.back();
  fl.pop_back();
  return id;
}

void Allocator::give(std::vector<int>& fl, int id) {
  // keep the stack sorted (descending), so the lowest free id is on top
  fl.insert(std::upper_bound(fl.begin(), fl.end(), id, [](int x, int y) { return x > y; }), id);
}

Allocator::Allocator(int slots_, int max_context_, int window_, int local_pages_, int global_pages_)
    : slots(slots_), max_context(max_context_), window(window_), local_pages(local_pages_),
      global_pages(global_pages_), seq(slots_) {
  for (int i = local_pages - 1; i >= 0; --i) free_local.push_back(i);
  for (int i = global_pages - 1; i >= 0; --i) free_global.push_back(i);
  const int max_pages = (max_context + kPage - 1) / kPage;
  for (auto& q : seq) {
    q.lpt.assign(max_pages, -1);
    q.gpt.assign(max_pages, -1);
  }
}

int Allocator::active() const {
  int n = 0;
  for (const auto& q : seq) n += q.used;
  return n;
}

// 1: admitted into *slot; 0: wait; -1: refused (never fits now and nothing runs)
int Allocator::admit(int total, int rows, int* slot) {
  *slot = -1;
  const int need_g = (total + kPage - 1) / kPage;
  const int need_l = local_reserve(total, rows);
  int free_slot = -1;
  for (int i = 0; i < slots && free_slot < 0; ++i)
    if (!seq[i].used) free_slot = i;
  if (free_slot >= 0 && reserved_l + need_l <= local_pages && reserved_g + need_g <= global_pages) {
    Seq& q = seq[free_slot];
    q.used = true;
    q.total = total;
    q.rows = rows;
    q.len = 0;
    q.first_query = 0;
    q.res_l = need_l;
    q.res_g = need_g;
    reserved_l += need_l;
    reserved_g += need_g;
    *slot = free_slot;
    return 1;
  }
  return active() == 0 ? -1 : 0;
}

// 0, or -1 (nothing changed) when a free list cannot supply the pages: the
// admission reservations make that impossible, so it means a broken
// invariant, reported rather than acted on.
int Allocator::extend(int slot, int new_len, int first_query) {
  Seq& q = seq[slot];
  const int last_page = (new_len - 1) / kPage;
  const int lo_page = std::max(0, first_query - window + 1) / kPage;
  int need_g = 0, need_l = 0, freed_l = 0;
  for (int i = 0; i <= last_page; ++i) {
    need_g += q.gpt[i] < 0;
    need_l += i >= lo_page && q.lpt[i] < 0;
    freed_l += i < lo_page && q.lpt[i] >= 0;
  }
  if (need_g > (int)free_global.size() || need_l > (int)free_local.size() + freed_l) return -1;
  for (int i = 0; i <= last_page; ++i) {
    if (q.gpt[i] < 0) q.gpt[i] = take(free_global);
  }
  for (int i = 0; i < lo_page; ++i)
    if (q.lpt[i] >= 0) {
      give(free_local, q.lpt[i]);
      q.lpt[i] = -1;
    }
  for (int i = lo_page; i <= last_page; ++i)
    if (q.lpt[i] < 0) q.lpt[i] = take(free_local);
  q.len = new_len;
  q.first_query = first_query;
  return 0;
}

void Allocator::release(int slot) {
  Seq& q = seq[slot];
  for (auto& id : q.lpt)
    if (id >= 0) {
      give(free_local, id);
      id = -1;
    }
  for (auto& id : q.gpt)
    if (id >= 0) {
      give(free_global, id);
      id = -1;
    }
  reserved_l -= q.res_l;
  reserved_g -= q.res_g;
  q = Seq{false, 0, 0, 0, 0, 0, 0, std::move(q.lpt), std::move(q.gpt)};
}

namespace {

// One workgroup per (page, 4 KiB piece): 256 lanes x 16 bytes.  Ids outside
// [0, num_pages) of their pool make the pair a no-op (the entry point has
// checked the host-visible geometry; the ids live on the device).
__global__ __launch_bounds__(256) void copy_pages_kernel(uint8_t* dst, const uint8_t* src, const int32_t* dst_pages,
                                                         const int32_t* src_pages, int64_t page_bytes,
                                                         int64_t dst_num_pages, int64_t src_num_pages) {
  const int i = blockIdx.y;
  const int64_t d = dst_pages[i], s = src_pages[i];
  if (d < 0 || d >= dst_num_pages || s < 0 || s >= src_num_pages) return;
  const int64_t off = (int64_t)blockIdx.x * 4096 + 16 * threadIdx.x;
  if (off >= page_bytes) return;
  const uint4 v = ld16(src + s * page_bytes + off);
  *reinterpret_cast<uint4*>(dst + d * page_bytes + off) = v;
}

}  // namespace

hipError_t launch_copy_pages(uint8_t* dst, const uint8_t* src, const int32_t* dst_pages, const int32_t* src_pages,
                             int n, int64_t page_bytes, int64_t dst_num_pages, int64_t src_num_pages,
                             hipStream_t stream) {
  dim3 grid((unsigned)((page_bytes + 4095) / 4096), (unsigned)n), block(256);
  hipLaunchKernelGGL(copy_pages_kernel, grid, block, 0, stream, dst, src, dst_pages, src_pages, page_bytes,
                     dst_num_pages, src_num_pages);
  return hipGetLastError();
}

}  // namespace gw
