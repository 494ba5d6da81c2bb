// C ABI of the gw library: argument validation (before any HIP call), split
// planning and kernel launches.  Declarations and contracts: include/gw.h.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "gw.h"
#include "gw_alloc.h"
#include "gw_kernels.h"
#include "gw_plan.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fn, const char* fmt, ...) {
  int n = snprintf(g_err, sizeof(g_err), "%s: ", fn);
  if (n < 0) n = 0;
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err + n, sizeof(g_err) - (size_t)n, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return GW_OK;
}

// The trace build's event buffer (gw_trace_buffer), else null.
uint64_t* g_trace = nullptr;

constexpr size_t kAlign = 256;
// Longest sequence served (tokens): keeps every page count and split bound
// of the plans well inside 32-bit arithmetic.
constexpr int kMaxSeqLen = 1 << 24;
// Most workgroups of one (1-D) launch.
constexpr long long kMaxGrid = 0x7fffffff;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool is_local(int f) { return f == GW_FAMILY_LOCAL; }
bool is_global(int f) { return f == GW_FAMILY_GLOBAL_COMPRESSED || f == GW_FAMILY_GLOBAL_FULL; }

// Geometry of a descriptor, without looking at base / num_pages.
int check_geometry(const gw_pool_desc* p, const char* fn) {
  if (!p) return fail(GW_ERR_INVALID_ARG, fn, "pool descriptor is null");
  if (!is_local(p->family) && !is_global(p->family))
    return fail(GW_ERR_INVALID_ARG, fn, "unknown family %d", p->family);
  switch (p->kv_dtype) {
    case GW_KV_BF16:
    case GW_KV_E4M3:
      break;
    default:
      return fail(GW_ERR_INVALID_ARG, fn, "unknown kv_dtype %d", p->kv_dtype);
  }
  if (p->page_size != 16) return fail(GW_ERR_GEOMETRY, fn, "page_size %d (must be 16)", p->page_size);
  if (is_local(p->family)) {
    if (p->head_dim != 256) return fail(GW_ERR_GEOMETRY, fn, "local head_dim %d (must be 256)", p->head_dim);
    if (p->rot_dim != 0 && p->rot_dim != 256)
      return fail(GW_ERR_GEOMETRY, fn, "local rot_dim %d (must be 256 or 0)", p->rot_dim);
    if (p->num_kv_heads < 1 || p->num_kv_heads > 65535)
      return fail(GW_ERR_GEOMETRY, fn, "local num_kv_heads %d", p->num_kv_heads);
  } else {
    if (p->head_dim != 512) return fail(GW_ERR_GEOMETRY, fn, "global head_dim %d (must be 512)", p->head_dim);
    if (p->rot_dim != 128) return fail(GW_ERR_GEOMETRY, fn, "global rot_dim %d (must be 128)", p->rot_dim);
    if (p->num_kv_heads != 1)
      return fail(GW_ERR_GEOMETRY, fn, "global num_kv_heads %d (must be 1)", p->num_kv_heads);
  }
  return GW_OK;
}

int64_t page_bytes_of(const gw_pool_desc* p) {
  const int64_t eb = p->kv_dtype == GW_KV_E4M3 ? 1 : 2;
  switch (p->family) {
    case GW_FAMILY_LOCAL: return 16LL * 2 * p->num_kv_heads * 256 * eb;
    case GW_FAMILY_GLOBAL_COMPRESSED: return 16LL * (512 + 128) * eb;
    case GW_FAMILY_GLOBAL_FULL: return 16LL * 1024 * eb;
  }
  return -1;
}

int check_pool(const gw_pool_desc* p, const char* fn) {
  int rc = check_geometry(p, fn);
  if (rc != GW_OK) return rc;
  if (!p->base) return fail(GW_ERR_INVALID_ARG, fn, "pool base is null");
  if (p->num_pages < 1) return fail(GW_ERR_INVALID_ARG, fn, "num_pages %lld", (long long)p->num_pages);
  return GW_OK;
}

// Largest split count of any decode row of a call.
// group: the call's query-group size (local family); the size query, which
// does not know it, passes 4, the size with the most splits.
int max_splits_for(int family, int max_seq_len, int window, int group) {
  if (family == GW_FAMILY_LOCAL) return gw::local_nsplit(gw::local_max_range_pages(max_seq_len, window), group);
  return gw::global_nsplit(gw::cdiv_i(max_seq_len, 16));
}

// Workspace: [split counters | call epochs (local) | partial accumulators |
// partial (max, sum)].  The counters must be zero before the first call (the
// caller zero-fills the workspace once); every call that completes leaves
// them zero again.  The local family's partials are (value, tag) pairs of 8
// bytes, tagged with the call's epoch (gw_local.hip); the global family's
// are plain fp32, reduced by a kernel of their own.
struct WsPlan {
  int max_splits;
  size_t counter_bytes, epoch_bytes, acc_bytes, ml_bytes, total;
};

WsPlan plan_workspace(int family, int num_seqs, int num_kv_heads, int num_q_heads, int head_dim,
                      int max_seq_len, int window, int group) {
  WsPlan w{};
  w.max_splits = max_splits_for(family, max_seq_len, window, group);
  if (w.max_splits <= 1 || num_seqs <= 0) return w;
  const bool local = family == GW_FAMILY_LOCAL;
  const size_t units = (size_t)num_seqs * num_q_heads * w.max_splits;
  const size_t elem = local ? sizeof(uint64_t) : sizeof(float);
  w.counter_bytes = align_up((size_t)num_seqs * num_kv_heads * sizeof(int));
  w.epoch_bytes = local ? align_up((size_t)num_seqs * num_kv_heads * sizeof(uint32_t)) : 0;
  w.acc_bytes = align_up(units * head_dim * elem);
  w.ml_bytes = align_up(units * 2 * elem);
  w.total = w.counter_bytes + w.epoch_bytes + w.acc_bytes + w.ml_bytes;
  return w;
}

// Compute units of the current device, read once per device (0 if the
// query fails).
int device_cus() {
  static std::mutex mu;
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = n;
  }
  return cus[dev];
}

// Consecutive splits of a (sequence, KV head) per local decode workgroup:
// the fewest (1, 2 or 4, up to gw::local_max_splits_per_wg) with which the
// launch needs no more workgroups than the device has CUs, and no more than
// the most splits a row has.  The plan and the arithmetic do not change
// with it (gw_local.hip), only how many workgroups carry the splits: a
// large batch runs fewer, longer workgroups, which merge their own splits
// in registers.
int local_splits_per_wg(long long pairs, int max_splits, int group, bool fp8) {
  const int cus = device_cus();
  const int most = gw::local_max_splits_per_wg(group, fp8);
  if (cus <= 0) return 1;
  int spw = 1;
  while (spw < most && spw < max_splits && pairs * gw::cdiv_i(max_splits, spw) > cus) spw *= 2;
  return spw;
}

// Arguments common to both attention entry points.
int check_attn_common(const char* fn, const void* q, int num_q_heads, const int32_t* q_indptr,
                      const int32_t* seq_lens, const int32_t* page_table, int pt_stride,
                      int num_seqs, int num_rows, int max_q_len, int max_seq_len, float scale,
                      const float* out) {
  if (num_seqs < 0 || num_seqs > 65535) return fail(GW_ERR_INVALID_ARG, fn, "num_seqs %d", num_seqs);
  if (num_rows < 0) return fail(GW_ERR_INVALID_ARG, fn, "num_rows %d", num_rows);
  if (num_q_heads < 1) return fail(GW_ERR_INVALID_ARG, fn, "num_q_heads %d", num_q_heads);
  if (max_q_len < 1) return fail(GW_ERR_INVALID_ARG, fn, "max_q_len %d", max_q_len);
  if (max_seq_len < 1 || max_seq_len > kMaxSeqLen)
    return fail(GW_ERR_INVALID_ARG, fn, "max_seq_len %d (served: 1 .. %d)", max_seq_len, kMaxSeqLen);
  if (max_q_len > max_seq_len)
    return fail(GW_ERR_INVALID_ARG, fn, "max_q_len %d exceeds max_seq_len %d", max_q_len, max_seq_len);
  if (!isfinite(scale)) return fail(GW_ERR_INVALID_ARG, fn, "scale is not finite");
  if (!q_indptr && num_rows != num_seqs)
    return fail(GW_ERR_INVALID_ARG, fn, "q_indptr is null but num_rows %d != num_seqs %d", num_rows, num_seqs);
  if (!q_indptr && max_q_len != 1)
    return fail(GW_ERR_INVALID_ARG, fn, "q_indptr is null but max_q_len %d != 1", max_q_len);
  if (pt_stride < gw::cdiv_i(max_seq_len, 16))
    return fail(GW_ERR_INVALID_ARG, fn, "pt_stride %d < pages of max_seq_len %d", pt_stride, max_seq_len);
  if (num_seqs == 0 || num_rows == 0) return GW_OK;
  if (!q || !seq_lens || !page_table || !out)
    return fail(GW_ERR_INVALID_ARG, fn, "null q, seq_lens, page_table or out");
  return GW_OK;
}

int hip_fail(const char* fn, hipError_t e) {
  return fail(GW_ERR_HIP, fn, "%s", hipGetErrorString(e));
}

}  // namespace

extern "C" {

#ifdef GW_TRACE
// Trace builds only (not part of the C ABI in gw.h): the device buffer of
// 16 x grid uint64 slots the decode kernels record their event times into
// (null: stop recording).
int gw_trace_buffer(void* dev_buf) {
  g_trace = static_cast<uint64_t*>(dev_buf);
  return GW_OK;
}
#endif


const char* gw_version(void) { return "gw 0.1.0 (gfx950, paged hybrid-KV decode attention)"; }

const char* gw_last_error(void) { return g_err; }

int64_t gw_pool_page_bytes(const gw_pool_desc* pool) {
  int rc = check_geometry(pool, "gw_pool_page_bytes");
  if (rc != GW_OK) return rc;
  ok();
  return page_bytes_of(pool);
}

int gw_rope_table(float* cos_out, float* sin_out, int32_t max_pos, int32_t rot_dim, int32_t head_dim,
                  double theta, void* stream) {
  const char* fn = "gw_rope_table";
  if (!cos_out || !sin_out) return fail(GW_ERR_INVALID_ARG, fn, "null output table");
  if (max_pos < 1) return fail(GW_ERR_INVALID_ARG, fn, "max_pos %d", max_pos);
  if (rot_dim < 2 || (rot_dim & 1) || rot_dim > head_dim)
    return fail(GW_ERR_INVALID_ARG, fn, "rot_dim %d with head_dim %d", rot_dim, head_dim);
  if (!(theta > 0.0) || !isfinite(theta)) return fail(GW_ERR_INVALID_ARG, fn, "theta must be > 0");
  hipError_t e = gw::launch_rope_table(cos_out, sin_out, max_pos, rot_dim, head_dim, theta,
                                       (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

int gw_kv_append(const gw_pool_desc* pool, const void* k_raw, const void* v, const int32_t* seq_idx,
                 const int32_t* pos, int32_t n_tok, const int32_t* page_table, int32_t pt_stride,
                 const float* rope_cos, const float* rope_sin, void* stream) {
  const char* fn = "gw_kv_append";
  int rc = check_pool(pool, fn);
  if (rc != GW_OK) return rc;
  if (n_tok < 0) return fail(GW_ERR_INVALID_ARG, fn, "n_tok %d", n_tok);
  if (pt_stride < 1) return fail(GW_ERR_INVALID_ARG, fn, "pt_stride %d", pt_stride);
  if ((rope_cos == nullptr) != (rope_sin == nullptr))
    return fail(GW_ERR_INVALID_ARG, fn, "rope_cos and rope_sin must both be set or both be null");
  const bool rope = rope_cos != nullptr;
  if (is_local(pool->family)) {
    if (pool->rot_dim == 0 && rope)
      return fail(GW_ERR_INVALID_ARG, fn, "rot_dim 0 takes no rotary tables");
    if (pool->rot_dim != 0 && !rope)
      return fail(GW_ERR_INVALID_ARG, fn, "rot_dim %d needs rotary tables", pool->rot_dim);
  } else {
    if (!rope) return fail(GW_ERR_INVALID_ARG, fn, "the global family needs rotary tables");
  }
  if (n_tok == 0) return ok();
  if (!v || !seq_idx || !pos || !page_table)
    return fail(GW_ERR_INVALID_ARG, fn, "null v, seq_idx, pos or page_table");
  if (is_local(pool->family) && !k_raw) return fail(GW_ERR_INVALID_ARG, fn, "k_raw is null");

  gw::AppendArgs a{};
  a.pool = static_cast<uint8_t*>(pool->base);
  a.page_bytes = page_bytes_of(pool);
  a.head_bytes = (int32_t)(a.page_bytes / pool->num_kv_heads);
  a.k_raw = static_cast<const uint16_t*>(k_raw);
  a.v = static_cast<const uint16_t*>(v);
  a.seq_idx = seq_idx;
  a.pos = pos;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.n_tok = n_tok;
  a.num_kv_heads = pool->num_kv_heads;
  hipError_t e;
  if (is_local(pool->family))
    e = gw::launch_append_local(a, pool->kv_dtype == GW_KV_E4M3, rope, (hipStream_t)stream);
  else
    e = gw::launch_append_global(a, pool->family == GW_FAMILY_GLOBAL_COMPRESSED, pool->kv_dtype == GW_KV_E4M3,
                                 (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

size_t gw_attn_workspace_bytes(int32_t family, int32_t num_seqs, int32_t num_rows, int32_t num_q_heads,
                               int32_t head_dim, int32_t max_seq_len, int32_t window, int32_t max_q_len) {
  (void)num_rows;
  (void)max_q_len;
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_seq_len <= 0) return 0;
  if (family == GW_FAMILY_LOCAL && window < 1) return 0;
  if (!is_local(family) && !is_global(family)) return 0;
  // one counter per (sequence, q head) bounds the per-(sequence, KV head) need
  return plan_workspace(family, num_seqs, num_q_heads, num_q_heads, head_dim, max_seq_len, window, 4).total;
}

}  // extern "C"

namespace {

// The allocation-free local entry point's workspace: one array per GPU, in
// the library's own device memory, held until the process ends.  Host code
// uses it only through the device address hipGetSymbolAddress returns for
// the current device (kept per device); the array's name is a host-side
// stand-in, not that address.
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array of the current device (its address resolved on the
// first call on that device), or an error status.
int scratch_for_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(fn, e);
  if (dev < 0 || dev >= kMaxDevices) return fail(GW_ERR_UNSUPPORTED, fn, "device %d (served: 0 .. %d)", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(fn, e);
    if (!ptr) return fail(GW_ERR_HIP, fn, "no device address for the scratch array");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GW_OK;
}

// Zero n bytes (a multiple of 16) at p: a plain fill kernel rather than a
// memset node, so that the call can be captured in a graph.
__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

int attn_local(const char* fn, const gw_pool_desc* pool, const void* q, int32_t num_q_heads,
               const void* k_new, const void* v_new, const float* rope_cos, const float* rope_sin,
               const int32_t* q_indptr, const int32_t* seq_lens, const int32_t* page_table, int32_t pt_stride,
               int32_t num_seqs, int32_t num_rows, int32_t max_q_len, int32_t max_seq_len, int32_t window,
               float scale, float* out, void* workspace, size_t workspace_bytes, bool noalloc, void* stream) {
  int rc = check_pool(pool, fn);
  if (rc != GW_OK) return rc;
  if (!is_local(pool->family))
    return fail(GW_ERR_INVALID_ARG, fn, "pool family %d is not GW_FAMILY_LOCAL", pool->family);
  if (window < 1) return fail(GW_ERR_INVALID_ARG, fn, "window %d (must be >= 1)", window);
  rc = check_attn_common(fn, q, num_q_heads, q_indptr, seq_lens, page_table, pt_stride, num_seqs,
                         num_rows, max_q_len, max_seq_len, scale, out);
  if (rc != GW_OK) return rc;
  if (num_q_heads % pool->num_kv_heads != 0)
    return fail(GW_ERR_GEOMETRY, fn, "num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
                pool->num_kv_heads);
  const int group = num_q_heads / pool->num_kv_heads;
  if (group != 1 && group != 2 && group != 4)
    return fail(GW_ERR_UNSUPPORTED, fn, "query group size %d (served: 1, 2, 4)", group);
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(GW_ERR_INVALID_ARG, fn, "k_new and v_new must both be set or both be null");
  if ((rope_cos == nullptr) != (rope_sin == nullptr))
    return fail(GW_ERR_INVALID_ARG, fn, "rope_cos and rope_sin must both be set or both be null");
  if (v_new && pool->rot_dim != 0 && !rope_cos)
    return fail(GW_ERR_INVALID_ARG, fn, "rot_dim %d needs rotary tables", pool->rot_dim);
  if (v_new && pool->rot_dim == 0 && rope_cos)
    return fail(GW_ERR_INVALID_ARG, fn, "rot_dim 0 takes no rotary tables");
  const WsPlan w = plan_workspace(GW_FAMILY_LOCAL, num_seqs, pool->num_kv_heads, num_q_heads, 256,
                                  max_seq_len, window, group);
  // grids: (split, KV head, sequence) for the decode rows, (row block, KV
  // head) for the prompt rows
  const int spw = local_splits_per_wg((long long)pool->num_kv_heads * num_seqs, std::max(w.max_splits, 1), group,
                                      pool->kv_dtype == GW_KV_E4M3);
  const long long dec_wgs = (long long)gw::cdiv_i(std::max(w.max_splits, 1), spw) * pool->num_kv_heads * num_seqs;
  // the prompt rows' own tokens are appended by workgroups after the decode items
  const long long app_units =
      v_new && max_q_len > 1
          ? gw::rows_append_items(num_rows, num_seqs, max_q_len) *
                gw::cdiv_i(pool->num_kv_heads, gw::kRowsAppendHeads)
          : 0;
  const int units_per_wg = 64 * gw::local_waves(group) / 256;
  if (app_units > kMaxGrid || dec_wgs + (app_units + units_per_wg - 1) / units_per_wg > kMaxGrid)
    return fail(GW_ERR_UNSUPPORTED, fn, "%lld decode workgroups and %lld append workgroups (served: up to %lld)",
                dec_wgs, (app_units + units_per_wg - 1) / units_per_wg, kMaxGrid);
  if (max_q_len > 1) {
    const long long pre_wgs =
        gw::prefill_items(num_rows, num_seqs, max_q_len, gw::local_prefill_rows(group)) * pool->num_kv_heads;
    if (pre_wgs > kMaxGrid)
      return fail(GW_ERR_UNSUPPORTED, fn, "%lld prompt-row workgroups (served: up to %lld)", pre_wgs, kMaxGrid);
  }
  if (noalloc) {
    if (w.total > kScratchBytes)
      return fail(GW_ERR_WORKSPACE, fn, "the call needs %zu bytes of scratch; this entry point holds %zu",
                  w.total, kScratchBytes);
  } else {
    if (workspace_bytes < w.total)
      return fail(GW_ERR_WORKSPACE, fn, "workspace %zu bytes < %zu needed", workspace_bytes, w.total);
    if (w.total > 0 && !workspace) return fail(GW_ERR_INVALID_ARG, fn, "workspace is null");
    if (w.total > 0 && ((uintptr_t)workspace % kAlign) != 0)
      return fail(GW_ERR_INVALID_ARG, fn, "workspace is not 256-byte aligned");
  }
  if (num_seqs == 0 || num_rows == 0) return ok();
  if (noalloc && w.total > 0) {
    // every call starts from a zeroed region: the split counters and call
    // epochs of the previous call (of any shape) sit elsewhere, and its
    // tagged partials must not pass for this call's
    rc = scratch_for_current_device(fn, &workspace);
    if (rc != GW_OK) return rc;
    (void)hipGetLastError();
    const size_t n16 = w.total / 16;   // the plan's regions are 256-byte multiples
    const unsigned blocks = (unsigned)std::min<size_t>((n16 + 255) / 256, 2048);
    hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<uint4*>(workspace), n16);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(fn, e);
  }

  gw::LocalAttnArgs a{};
  a.trace = g_trace;
  a.pool = static_cast<const uint8_t*>(pool->base);
  a.page_bytes = page_bytes_of(pool);
  a.head_bytes = (int32_t)(a.page_bytes / pool->num_kv_heads);
  a.q = static_cast<const uint16_t*>(q);
  a.q_indptr = q_indptr;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.window = window;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.counters = w.total ? reinterpret_cast<int*>(ws) : nullptr;
  a.epochs = w.total ? reinterpret_cast<uint32_t*>(ws + w.counter_bytes) : nullptr;
  a.part_acc = w.total ? reinterpret_cast<uint64_t*>(ws + w.counter_bytes + w.epoch_bytes) : nullptr;
  a.part_ml = w.total ? reinterpret_cast<uint64_t*>(ws + w.counter_bytes + w.epoch_bytes + w.acc_bytes) : nullptr;
  a.max_splits = std::max(w.max_splits, 1);
  a.splits_per_wg = spw;
  a.num_seqs = num_seqs;
  a.num_rows = num_rows;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.append_units = (int32_t)app_units;
  (void)hipGetLastError();   // a stale error from earlier work is not ours to report
  const bool fp8 = pool->kv_dtype == GW_KV_E4M3;
  hipError_t e;
  // the decode rows (each appending its own token) and the prompt rows'
  // append in one launch; the prompt rows attend in the next
  e = gw::launch_local_decode(a, group, fp8, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  if (max_q_len > 1) {
    e = gw::launch_local_prefill(a, group, fp8, max_q_len, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
  }
  return ok();
}

}  // namespace

extern "C" {

int gw_decode_attn_local(const gw_pool_desc* pool, const void* q, int32_t num_q_heads,
                         const void* k_new, const void* v_new, const float* rope_cos,
                         const float* rope_sin, const int32_t* q_indptr, const int32_t* seq_lens, const int32_t* page_table,
                         int32_t pt_stride, int32_t num_seqs, int32_t num_rows, int32_t max_q_len,
                         int32_t max_seq_len, int32_t window, float scale, float* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return attn_local("gw_decode_attn_local", pool, q, num_q_heads, k_new, v_new, rope_cos, rope_sin, q_indptr,
                    seq_lens, page_table, pt_stride, num_seqs, num_rows, max_q_len, max_seq_len, window, scale,
                    out, workspace, workspace_bytes, false, stream);
}

int gw_decode_attn_local_noalloc(const gw_pool_desc* pool, const void* q, int32_t num_q_heads,
                                 const void* k_new, const void* v_new, const float* rope_cos,
                                 const float* rope_sin, const int32_t* q_indptr, const int32_t* seq_lens,
                                 const int32_t* page_table, int32_t pt_stride, int32_t num_seqs,
                                 int32_t num_rows, int32_t max_q_len, int32_t max_seq_len, int32_t window,
                                 float scale, float* out, void* stream) {
  return attn_local("gw_decode_attn_local_noalloc", pool, q, num_q_heads, k_new, v_new, rope_cos, rope_sin,
                    q_indptr, seq_lens, page_table, pt_stride, num_seqs, num_rows, max_q_len, max_seq_len, window,
                    scale, out, nullptr, 0, true, stream);
}

int gw_decode_attn_global(const gw_pool_desc* pool, const void* q, int32_t num_q_heads,
                          const void* k_new, const void* v_new, const float* rope_cos, const float* rope_sin,
                          const int32_t* q_indptr, const int32_t* seq_lens, const int32_t* page_table,
                          int32_t pt_stride, int32_t num_seqs, int32_t num_rows, int32_t max_q_len,
                          int32_t max_seq_len, float scale, float* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  const char* fn = "gw_decode_attn_global";
  int rc = check_pool(pool, fn);
  if (rc != GW_OK) return rc;
  if (!is_global(pool->family))
    return fail(GW_ERR_INVALID_ARG, fn, "pool family %d is not a global family", pool->family);
  rc = check_attn_common(fn, q, num_q_heads, q_indptr, seq_lens, page_table, pt_stride, num_seqs,
                         num_rows, max_q_len, max_seq_len, scale, out);
  if (rc != GW_OK) return rc;
  if (num_q_heads != 16 && num_q_heads != 32)
    return fail(GW_ERR_UNSUPPORTED, fn, "num_q_heads %d (served: 16, 32)", num_q_heads);
  const bool fp8 = pool->kv_dtype == GW_KV_E4M3;
  if ((rope_cos == nullptr) != (rope_sin == nullptr))
    return fail(GW_ERR_INVALID_ARG, fn, "rope_cos and rope_sin must both be set or both be null");
  if (v_new && !rope_cos) return fail(GW_ERR_INVALID_ARG, fn, "the global family needs rotary tables");
  if (k_new && !v_new) return fail(GW_ERR_INVALID_ARG, fn, "k_new is set but v_new is null");
  const WsPlan w = plan_workspace(pool->family, num_seqs, 1, num_q_heads, 512, max_seq_len, 0, 1);
  // the prompt rows' own tokens are appended by workgroups after the decode items, two units each
  const long long app_units = v_new && max_q_len > 1 ? gw::rows_append_items(num_rows, num_seqs, max_q_len) : 0;
  if ((long long)w.max_splits * num_seqs + (app_units + 1) / 2 > kMaxGrid)
    return fail(GW_ERR_UNSUPPORTED, fn, "%lld decode workgroups and %lld append workgroups (served: up to %lld)",
                (long long)w.max_splits * num_seqs, (app_units + 1) / 2, kMaxGrid);
  if (max_q_len > 1) {
    // the decode rows' reduce (two units of 256 threads per workgroup), then the prompt rows' items
    const long long pre_wgs = gw::prefill_items(num_rows, num_seqs, max_q_len, gw::global_prefill_rows(num_q_heads)) +
                              (w.max_splits > 1 ? ((long long)num_seqs * gw::reduce_groups(num_q_heads) + 1) / 2 : 0);
    if (pre_wgs > kMaxGrid)
      return fail(GW_ERR_UNSUPPORTED, fn, "%lld prompt-row workgroups (served: up to %lld)", pre_wgs, kMaxGrid);
  }
  if (workspace_bytes < w.total)
    return fail(GW_ERR_WORKSPACE, fn, "workspace %zu bytes < %zu needed", workspace_bytes, w.total);
  if (w.total > 0 && !workspace) return fail(GW_ERR_INVALID_ARG, fn, "workspace is null");
  if (w.total > 0 && ((uintptr_t)workspace % kAlign) != 0)
    return fail(GW_ERR_INVALID_ARG, fn, "workspace is not 256-byte aligned");
  if (num_seqs == 0 || num_rows == 0) return ok();

  gw::GlobalAttnArgs a{};
  a.trace = g_trace;
  a.pool = static_cast<const uint8_t*>(pool->base);
  a.page_bytes = page_bytes_of(pool);
  a.q = static_cast<const uint16_t*>(q);
  a.q_indptr = q_indptr;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.num_q_heads = num_q_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.counters = w.total ? reinterpret_cast<int*>(ws) : nullptr;
  a.part_acc = w.total ? reinterpret_cast<float*>(ws + w.counter_bytes) : nullptr;
  a.part_ml = w.total ? reinterpret_cast<float*>(ws + w.counter_bytes + w.acc_bytes) : nullptr;
  a.max_splits = w.max_splits;
  a.num_seqs = num_seqs;
  a.num_rows = num_rows;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.append_units = (int32_t)app_units;
  (void)hipGetLastError();
  const bool compressed = pool->family == GW_FAMILY_GLOBAL_COMPRESSED;
  hipError_t e;
  // the decode rows (each appending its own token) and the prompt rows'
  // append in one launch; then the prompt rows' attention and the decode
  // rows' cross-split reduce in one launch, or the reduce alone
  e = gw::launch_global_decode(a, compressed, fp8, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  if (max_q_len > 1) {
    e = gw::launch_global_prefill(a, compressed, fp8, max_q_len, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
  } else if (w.max_splits > 1) {
    gw::ReduceArgs r{q_indptr, seq_lens, a.part_acc, a.part_ml, out, num_q_heads, w.max_splits};
    e = gw::launch_split_reduce(r, num_seqs, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
  }
  return ok();
}

// ------------------------------------------------------ pool lifecycle --
struct gw_page_alloc {
  gw::Allocator impl;
};

int gw_alloc_create(int32_t slots, int32_t max_context, int32_t window, int32_t local_pages,
                    int32_t global_pages, gw_page_alloc** out) {
  const char* fn = "gw_alloc_create";
  if (!out) return fail(GW_ERR_INVALID_ARG, fn, "out is null");
  *out = nullptr;
  if (slots < 1 || slots > (1 << 20)) return fail(GW_ERR_INVALID_ARG, fn, "slots %d", slots);
  if (max_context < 1 || max_context > (1 << 24)) return fail(GW_ERR_INVALID_ARG, fn, "max_context %d", max_context);
  if (window < 1) return fail(GW_ERR_INVALID_ARG, fn, "window %d", window);
  if (local_pages < 0 || global_pages < 0)
    return fail(GW_ERR_INVALID_ARG, fn, "page counts %d, %d", local_pages, global_pages);
  if ((int64_t)slots * ((max_context + 15) / 16) > (1LL << 28))
    return fail(GW_ERR_INVALID_ARG, fn, "slots x pages per slot too large");
  try {
    *out = new gw_page_alloc{gw::Allocator(slots, max_context, window, local_pages, global_pages)};
  } catch (...) {
    return fail(GW_ERR_INVALID_ARG, fn, "out of host memory");
  }
  return ok();
}

int gw_alloc_destroy(gw_page_alloc* a) {
  delete a;
  return ok();
}

int gw_alloc_admit(gw_page_alloc* a, int32_t total_tokens, int32_t max_step_rows, int32_t* slot) {
  const char* fn = "gw_alloc_admit";
  if (!a || !slot) return fail(GW_ERR_INVALID_ARG, fn, "null allocator or slot");
  *slot = -1;
  gw::Allocator& A = a->impl;
  if (total_tokens < 1) return fail(GW_ERR_INVALID_ARG, fn, "total_tokens %d", total_tokens);
  if (max_step_rows < 1 || max_step_rows > total_tokens)
    return fail(GW_ERR_INVALID_ARG, fn, "max_step_rows %d (1 .. total_tokens)", max_step_rows);
  if (total_tokens > A.max_context)
    return fail(GW_ERR_REFUSED, fn, "total_tokens %d exceeds the ceiling %d", total_tokens, A.max_context);
  const int r = A.admit(total_tokens, max_step_rows, slot);
  if (r < 0) return fail(GW_ERR_REFUSED, fn, "the pools cannot hold the request and nothing else runs");
  return ok();
}

int gw_alloc_extend(gw_page_alloc* a, int32_t slot, int32_t new_len, int32_t first_query_pos) {
  const char* fn = "gw_alloc_extend";
  if (!a) return fail(GW_ERR_INVALID_ARG, fn, "allocator is null");
  gw::Allocator& A = a->impl;
  if (slot < 0 || slot >= A.slots || !A.seq[slot].used) return fail(GW_ERR_INVALID_ARG, fn, "slot %d is not active", slot);
  const auto& q = A.seq[slot];
  if (new_len < std::max(1, q.len) || new_len > q.total)
    return fail(GW_ERR_INVALID_ARG, fn, "new_len %d (%d .. %d)", new_len, std::max(1, q.len), q.total);
  if (first_query_pos < q.first_query || first_query_pos > new_len - 1)
    return fail(GW_ERR_INVALID_ARG, fn, "first_query_pos %d (%d .. %d)", first_query_pos, q.first_query, new_len - 1);
  if (new_len - first_query_pos > q.rows)
    return fail(GW_ERR_INVALID_ARG, fn, "%d rows in one step > max_step_rows %d", new_len - first_query_pos, q.rows);
  if (A.extend(slot, new_len, first_query_pos) != 0)
    return fail(GW_ERR_REFUSED, fn, "a free list cannot supply the pages (the reservations do not cover them)");
  return ok();
}

int gw_alloc_release(gw_page_alloc* a, int32_t slot) {
  const char* fn = "gw_alloc_release";
  if (!a) return fail(GW_ERR_INVALID_ARG, fn, "allocator is null");
  if (slot < 0 || slot >= a->impl.slots || !a->impl.seq[slot].used)
    return fail(GW_ERR_INVALID_ARG, fn, "slot %d is not active", slot);
  a->impl.release(slot);
  return ok();
}

int gw_alloc_tables(const gw_page_alloc* a, int32_t* local_pt, int32_t local_stride, int32_t* global_pt,
                    int32_t global_stride, int32_t* seq_lens) {
  const char* fn = "gw_alloc_tables";
  if (!a || !local_pt || !global_pt) return fail(GW_ERR_INVALID_ARG, fn, "null allocator or table");
  const gw::Allocator& A = a->impl;
  const int np = (A.max_context + 15) / 16;
  if (local_stride < np || global_stride < np)
    return fail(GW_ERR_INVALID_ARG, fn, "strides %d, %d < %d pages", local_stride, global_stride, np);
  for (int s = 0; s < A.slots; ++s) {
    const auto& q = A.seq[s];
    for (int i = 0; i < local_stride; ++i) local_pt[(int64_t)s * local_stride + i] = i < np ? q.lpt[i] : -1;
    for (int i = 0; i < global_stride; ++i) global_pt[(int64_t)s * global_stride + i] = i < np ? q.gpt[i] : -1;
    if (seq_lens) seq_lens[s] = q.used ? q.len : 0;
  }
  return ok();
}

int gw_alloc_stats(const gw_page_alloc* a, int32_t* stats) {
  if (!a || !stats) return fail(GW_ERR_INVALID_ARG, "gw_alloc_stats", "null allocator or stats");
  const gw::Allocator& A = a->impl;
  stats[0] = (int32_t)A.free_local.size();
  stats[1] = (int32_t)A.free_global.size();
  stats[2] = A.reserved_l;
  stats[3] = A.reserved_g;
  stats[4] = A.active();
  stats[5] = A.slots;
  return ok();
}

int gw_copy_pages(const gw_pool_desc* dst, const gw_pool_desc* src, const int32_t* dst_pages,
                  const int32_t* src_pages, int32_t n, void* stream) {
  const char* fn = "gw_copy_pages";
  int rc = check_pool(dst, fn);
  if (rc != GW_OK) return rc;
  rc = check_pool(src, fn);
  if (rc != GW_OK) return rc;
  if (dst->family != src->family || dst->kv_dtype != src->kv_dtype || page_bytes_of(dst) != page_bytes_of(src))
    return fail(GW_ERR_GEOMETRY, fn, "the two pools differ in family, dtype or page size");
  if (n < 0) return fail(GW_ERR_INVALID_ARG, fn, "n %d", n);
  if (n == 0) return ok();
  if (!dst_pages || !src_pages) return fail(GW_ERR_INVALID_ARG, fn, "null page list");
  (void)hipGetLastError();
  for (int32_t c = 0; c < n; c += 65535) {
    const int m = std::min(65535, n - c);
    hipError_t e = gw::launch_copy_pages(static_cast<uint8_t*>(dst->base), static_cast<const uint8_t*>(src->base),
                                         dst_pages + c, src_pages + c, m, page_bytes_of(dst), dst->num_pages,
                                         src->num_pages, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
  }
  return ok();
}

}  // extern "C"
