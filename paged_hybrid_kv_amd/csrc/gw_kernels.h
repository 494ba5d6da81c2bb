// Internal launch interface between the C ABI (gw_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gw {

struct LocalAttnArgs {
  const uint8_t* pool;        // page 0 of the layer's local pool
  int64_t page_bytes;         // bytes per physical page
  int32_t head_bytes;         // bytes per (page, KV head): K block + V block
  const uint16_t* q;          // bf16 [rows][Hq][256]
  const int32_t* q_indptr;    // [S+1] or null (one row per sequence)
  const int32_t* seq_lens;    // [S]
  const int32_t* page_table;  // [S][pt_stride]
  int32_t pt_stride;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t window;
  float scale_log2;           // softmax scale * log2(e)
  float* out;                 // fp32 [rows][Hq][256]
  // split partials as (fp32 value | tag << 32) pairs, tag = the call's epoch + 1
  uint64_t* part_acc;         // [S][Hq][max_splits][256]
  uint64_t* part_ml;          // [S][Hq][max_splits][2]: (max, sum) in base 2
  int* counters;              // [S][Hkv] splits finished; zero between calls
  uint32_t* epochs;           // [S][Hkv] calls with split partials so far
  int32_t max_splits;
  int32_t splits_per_wg;      // consecutive splits of a (sequence, KV head) per workgroup: 1, 2 or 4
  int32_t num_seqs;
  int32_t num_rows;
  const uint16_t* k_new;      // bf16 [rows][Hkv][256] raw K of each row's own token, or null
  const uint16_t* v_new;      // bf16 [rows][Hkv][256], or null (no append)
  const float* rope_cos;      // [max_pos][128] or null (K stored as given)
  const float* rope_sin;
  // the prompt rows' own tokens: append units (page item x block of two KV
  // heads) taken by the decode kernel's workgroups from append_wg0 on, 256
  // threads a unit; 0 when the call appends none
  int32_t append_units;
  int32_t append_wg0;
  uint64_t* trace;            // per-workgroup event times (trace builds only), else null
};

struct GlobalAttnArgs {
  const uint8_t* pool;
  int64_t page_bytes;         // 20480 compressed, 32768 full
  const uint16_t* q;          // bf16 [rows][Hq][512]
  const int32_t* q_indptr;
  const int32_t* seq_lens;
  const int32_t* page_table;
  int32_t pt_stride;
  int32_t num_q_heads;        // 16 or 32
  float scale_log2;
  float* out;                 // fp32 [rows][Hq][512]
  float* part_acc;            // fp32 [S][max_splits][Hq / 16][32 blocks][64 lanes][4] (MFMA fragment order)
  float* part_ml;             // fp32 [S][max_splits][Hq][2]
  int* counters;              // [S] splits finished; zero between calls
  int32_t max_splits;
  int32_t num_seqs;
  int32_t num_rows;
  const uint16_t* k_new;      // bf16 [rows][512] raw K of each row's token (dims 0..127 read), or null: K = V
  const uint16_t* v_new;      // bf16 [rows][512] raw V of each row's token, or null
  const float* rope_cos;      // [max_pos][64]
  const float* rope_sin;
  // the prompt rows' own tokens: append units (one page item each) taken by
  // the decode kernel's workgroups from append_wg0 on, 256 threads a unit;
  // 0 when the call appends none
  int32_t append_units;
  int32_t append_wg0;
  // calls with prompt rows: the decode rows' cross-split reduce runs in the
  // prompt-row kernel's first reduce_wgs workgroups
  int32_t reduce_wgs;
  uint64_t* trace;            // per-workgroup event times (trace builds only), else null
};

// Global family's cross-split reduce (gw_global.hip).
struct ReduceArgs {
  const int32_t* q_indptr;
  const int32_t* seq_lens;
  const float* part_acc;      // fp32 [S][max_splits][Hq / 16][32 blocks][64 lanes][4]
  const float* part_ml;       // fp32 [S][max_splits][Hq][2]
  float* out;                 // fp32 [rows][Hq][512]
  int32_t num_q_heads;
  int32_t max_splits;
};

struct AppendArgs {
  uint8_t* pool;
  int64_t page_bytes;
  int32_t head_bytes;         // local: bytes per (page, KV head)
  const uint16_t* k_raw;      // bf16 [n][Hkv][D] (local only)
  const uint16_t* v;          // bf16 [n][Hkv][D]
  const int32_t* seq_idx;
  const int32_t* pos;
  const int32_t* page_table;
  int32_t pt_stride;
  const float* rope_cos;      // [max_pos][rot/2] or null
  const float* rope_sin;
  int32_t n_tok;
  int32_t num_kv_heads;
  // Rows mode (the prompt rows of an attention call, gw_rows_append.h):
  // token i is query row i of the call -- its sequence found in q_indptr
  // (or i itself when q_indptr is null: one row per sequence), its position
  // seq_lens[s] - q_len + (i - q_indptr[s]); seq_idx / pos are unused.
  // skip_single: leave out the rows of one-row sequences (their decode
  // kernel appends them).  The per-token kernels take seq_idx / pos.
  const int32_t* q_indptr;
  const int32_t* seq_lens;
  int32_t num_seqs;
  int32_t skip_single;
};

// Each launcher enqueues its kernel(s) on `stream` and returns the
// hipGetLastError() status of the launch.
hipError_t launch_local_decode(const LocalAttnArgs& a, int group, bool fp8, hipStream_t stream);
hipError_t launch_global_decode(const GlobalAttnArgs& a, bool compressed, bool fp8, hipStream_t stream);
hipError_t launch_local_prefill(const LocalAttnArgs& a, int group, bool fp8, int max_q_len,
                                hipStream_t stream);
hipError_t launch_global_prefill(const GlobalAttnArgs& a, bool compressed, bool fp8, int max_q_len,
                                 hipStream_t stream);
hipError_t launch_split_reduce(const ReduceArgs& a, int num_seqs, hipStream_t stream);
hipError_t launch_append_local(const AppendArgs& a, bool fp8, bool rope, hipStream_t stream);
// Rows mode (seq_lens set): one workgroup per (sequence, page of its rows).
hipError_t launch_append_global(const AppendArgs& a, bool compressed, bool fp8, hipStream_t stream);
hipError_t launch_rope_table(float* cos_out, float* sin_out, int max_pos, int rot_dim,
                             int head_dim, double theta, hipStream_t stream);

}  // namespace gw
