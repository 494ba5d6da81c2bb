/*
 * gw.h -- paged hybrid-KV decode attention for MI355X (gfx950), C ABI.
 *
 * The operation: batched attention of query rows over paged KV caches of
 * the two attention families of the Gemma 4 hybrid stack (pegainfer
 * "Gemma 4" page, intro and Architecture notes):
 *   - local layers: sliding window (1024 tokens), head dim 256, grouped
 *     query heads (16 q heads over 8 KV heads), K rotated on all 256 dims
 *     (theta 1e4); K/V stored as bf16, or as e4m3 at scale 1.0 (pegainfer
 *     PR #1012, Description);
 *   - global layers: whole context, head dim 512, one KV head shared by
 *     every q head; K and V are tied and only the first 128 dims of K are
 *     rotated (theta 1e6, frequency denominator 512), so a page may store V
 *     plus the rotated quarter of K only -- 0.625x the bytes -- and K is
 *     rebuilt exactly inside the kernel (Gewell post, "the Why").
 * Both families use 16-token pages and one page table each (pegainfer
 * "Gemma 4" page, Scheduling).
 *
 * Conventions for every entry point:
 *   - All pointer arguments are DEVICE pointers unless marked (host).
 *   - The caller owns all memory: the library never allocates or frees
 *     device memory and never synchronizes.  Work is enqueued on `stream`
 *     (a hipStream_t passed as void*; NULL = the legacy default stream).
 *     (One exception: gw_decode_attn_local_noalloc keeps its workspace in a
 *     static device array of the library's own.)
 *   - Every host-checkable argument is validated before any HIP call; a
 *     rejected call returns a negative gw_status and launches nothing.
 *   - gw_last_error() then holds a message that starts with the name of the
 *     entry point that ran (thread-local; valid until the next call on the
 *     same thread).
 *   - Device-resident preconditions are the caller's contract and are not
 *     checked: seq_lens[s] >= 1; every page a call touches has a valid
 *     page-table entry in [0, num_pages); no two tokens of one append call
 *     write the same slot; positions < the rotary table length.
 *   - Reentrant; no mutable global state beyond the thread-local message
 *     (and the per-device address of gw_decode_attn_local_noalloc's array).
 */
#ifndef GW_H
#define GW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
typedef enum gw_status {
  GW_OK = 0,
  GW_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad enum value   */
  GW_ERR_UNSUPPORTED = -2, /* valid but not served (e.g. group size > 8)     */
  GW_ERR_GEOMETRY = -3,    /* shape does not match the family's layout      */
  GW_ERR_WORKSPACE = -4,   /* workspace smaller than gw_attn_workspace_bytes */
  GW_ERR_HIP = -5,         /* a HIP launch failed; message has the reason   */
  GW_ERR_REFUSED = -6      /* admission refused: the request can never run  */
} gw_status;

/* --------------------------------------------------------------- enums -- */
/* No zero value on purpose: an unset field is rejected, never defaulted. */
typedef enum gw_family {
  GW_FAMILY_LOCAL = 1,             /* sliding-window local layers           */
  GW_FAMILY_GLOBAL_COMPRESSED = 2, /* global layers, V + rotated K quarter  */
  GW_FAMILY_GLOBAL_FULL = 3        /* global layers, full K and V records   */
} gw_family;

typedef enum gw_kv_dtype {
  GW_KV_BF16 = 1, /* 2-byte bfloat16                                        */
  GW_KV_E4M3 = 2  /* 1-byte OCP e4m3 (E4M3FN), scale 1.0                    */
} gw_kv_dtype;

/* ------------------------------------------------------------ the pool -- */
/*
 * One layer's paged KV pool.  `base` points at num_pages * page_bytes bytes
 * (gw_pool_page_bytes).  Logical token t of a sequence lives in physical page
 * page_table[seq * pt_stride + t / 16] at slot t % 16.
 *
 * Geometry served:
 *   LOCAL:             page_size 16, head_dim 256, rot_dim 256 (or 0 = K is
 *                      stored as given), num_kv_heads >= 1, bf16 or e4m3.
 *   GLOBAL_COMPRESSED: page_size 16, head_dim 512, rot_dim 128, one KV head,
 *                      bf16 or e4m3.
 *   GLOBAL_FULL:       as GLOBAL_COMPRESSED.
 *
 * Element order inside a page (elements of kv_dtype):
 *   LOCAL page = [num_kv_heads][K block, V block], block = 16 x 256:
 *     bf16 K: element ((k*16 + t)*4 + c)*8 + e   holds K[t][64c + 8k + e]
 *             (k < 8, t < 16, c < 4, e < 8)
 *     bf16 V: element ((u*64 + l)*4 + j)*2 + i   holds V[2u + i][4l + j]
 *             (u < 8, l < 64, j < 4, i < 2)
 *     e4m3 K: element ((k*16 + t)*4 + c)*16 + e  holds K[t][64c + 16k + e]
 *             (k < 4, t < 16, c < 4, e < 16)
 *     e4m3 V: element ((u*64 + l)*4 + j)*4 + i   holds V[4u + i][4l + j]
 *             (u < 4, l < 64, j < 4, i < 4)
 *   GLOBAL_COMPRESSED page = V block [16][512], then K_rot block [16][128]
 *   GLOBAL_FULL page       = K block [16][512], then V block [16][512]
 *     each block chunk-major, a chunk being 16 bytes of one token:
 *     bf16: element (c*16 + t)*8 + e   holds X[t][8c + e]
 *     e4m3: element (c*16 + t)*16 + e  holds X[t][16c + e]
 *   (page bytes: compressed 20480 bf16 / 10240 e4m3, full 32768 / 16384)
 * (The orders put the 16 bytes one GPU lane loads next to the 16 bytes its
 * neighbour lane loads, so every page is read with whole 1 KiB wave loads.)
 */
typedef struct gw_pool_desc {
  int32_t family;       /* gw_family                                      */
  int32_t kv_dtype;     /* gw_kv_dtype                                    */
  int32_t page_size;    /* tokens per page; must be 16                    */
  int32_t num_kv_heads; /* local: >= 1; global: 1                         */
  int32_t head_dim;     /* local: 256; global: 512                        */
  int32_t rot_dim;      /* rotated dims of K: local 256 or 0; global 128  */
  int64_t num_pages;    /* physical pages behind base                     */
  void* base;           /* device pointer to page 0                       */
} gw_pool_desc;

/* ------------------------------------------------------------- queries -- */
/* Library version string (static storage). */
const char* gw_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char* gw_last_error(void);

/*
 * Bytes of one physical page of `pool` (host-only; no HIP call), or a
 * negative gw_status if the descriptor is invalid.  LOCAL: 16 * 2 *
 * num_kv_heads * 256 * elem_bytes; GLOBAL_COMPRESSED: 16 * 640 * 2;
 * GLOBAL_FULL: 16 * 1024 * 2 (Gewell post, "the Why": 640/1024 = 0.625).
 */
int64_t gw_pool_page_bytes(const gw_pool_desc* pool /* host */);

/* --------------------------------------------------------- rotary table -- */
/*
 * Fill cos/sin tables for RoPE (pegainfer "Gemma 4" page, Architecture
 * notes: local "full 256, theta 10k"; global "proportional 128/512, theta
 * 1M", the frequency denominator staying the full head dimension):
 *   cos_out[p * (rot_dim/2) + i] = cos(p * theta^(-2i/head_dim)), i < rot_dim/2
 *   sin_out[...]                 = sin(...)
 * for p in [0, max_pos), computed in fp64 on the device, stored as fp32.
 * rot_dim even, 2 <= rot_dim <= head_dim, theta > 0, max_pos >= 1.
 */
int gw_rope_table(float* cos_out, float* sin_out, int32_t max_pos, int32_t rot_dim,
                  int32_t head_dim, double theta, void* stream);

/* --------------------------------------------------------------- append -- */
/*
 * Write n_tok new tokens' K/V into `pool` (the prep step before attention:
 * pegainfer PR #1012, Description -- the prep kernel rotates and stores K/V
 * with the store type as a parameter; Gewell post, "the Why" -- the global
 * record is V plus the rotated quarter of K).
 *
 *   k_raw : bf16 [n_tok][num_kv_heads][head_dim], K before rotation.
 *           LOCAL: required.  GLOBAL families: optional -- NULL when K is V
 *           before rotation (the tied store); otherwise only its first 128
 *           dims are read, the quarter that rotates into K_rot.  The record
 *           keeps V for dims 128..511 in both global layouts, so a model whose
 *           K there is V * w_k (a per-dim norm weight on K: Gewell post, "the
 *           Why" -- only the rotated quarter differs in what is stored) passes
 *           q with dims 128..511 multiplied by w_k to the attention call,
 *           which gives the same scores.
 *   v     : bf16 [n_tok][num_kv_heads][head_dim].
 *   seq_idx, pos : int32 [n_tok]; token i goes to sequence seq_idx[i] at
 *           position pos[i], i.e. page page_table[seq_idx[i]*pt_stride +
 *           pos[i]/16], slot pos[i] % 16.
 *   rope_cos, rope_sin : fp32 [max_pos][rot_dim/2] from gw_rope_table, or
 *           both NULL to store K unrotated (LOCAL with rot_dim 0 requires
 *           NULL; rot_dim > 0 requires tables).
 * Per element, in fp32: rotate the first rot_dim dims of K as pairs
 * (i, i + rot_dim/2) by angle pos*inv_freq_i:
 *   y_i = x_i*cos - x_{i+R/2}*sin,  y_{i+R/2} = x_{i+R/2}*cos + x_i*sin,
 * round to bf16 (nearest-even); for e4m3 round that bf16 value once more to
 * e4m3 (nearest-even, saturating to +-448, NaN kept).
 *   LOCAL:             K block <- rotated K, V block <- V.
 *   GLOBAL_COMPRESSED: V block <- V, K_rot block <- rotated K[0:128]
 *                      (K = k_raw, or V when k_raw is NULL).
 *   GLOBAL_FULL:       K block <- [rotated K[0:128], V[128:512]], V <- V.
 * For an e4m3 pool every stored element, K_rot and V alike, is the e4m3
 * code of the bf16 record element.  n_tok == 0 is a no-op returning GW_OK.
 */
int gw_kv_append(const gw_pool_desc* pool /* host */, const void* k_raw, const void* v,
                 const int32_t* seq_idx, const int32_t* pos, int32_t n_tok,
                 const int32_t* page_table, int32_t pt_stride, const float* rope_cos,
                 const float* rope_sin, void* stream);

/* ------------------------------------------------------------ attention -- */
/*
 * Query rows and sequences (pegainfer "Gemma 4" page, Scheduling: every
 * active request advances one token per step, and a new prompt's rows are
 * computed in the same step):
 *   num_seqs sequences; sequence s has seq_lens[s] tokens (its current tokens
 *   included) and q_len_s = q_indptr[s+1] - q_indptr[s] query rows, rows
 *   q_indptr[s] .. q_indptr[s+1]-1, the last q_len_s tokens of the sequence:
 *   row r of s is at position seq_lens[s] - q_len_s + r.
 *   q_indptr NULL means one row per sequence (num_rows == num_seqs).
 *   A row at position p attends keys j with lo <= j <= p, lo = max(0,
 *   p - window + 1) for LOCAL and 0 for GLOBAL; q head h reads KV head
 *   h / (num_q_heads / num_kv_heads).
 *   out[row][h][:] = sum_j softmax_j(scale * q[row][h] . K[j]) V[j], fp32.
 * Host sizing arguments (upper bounds used to size grids; a device value
 * beyond them is a contract violation): num_rows = q_indptr[num_seqs];
 * max_q_len >= every q_len_s; max_seq_len >= every seq_lens[s];
 * max_seq_len <= 2^24 (16,777,216 tokens).
 *
 *   q   : bf16 [num_rows][num_q_heads][head_dim], already rotated.
 *   out : fp32 [num_rows][num_q_heads][head_dim].
 *   k_new, v_new, rope_cos, rope_sin : optional append of each row's own
 *     token before attention, with exactly gw_kv_append's arithmetic and
 *     placement (the prep step fused into the call): k_new/v_new hold the
 *     raw K/V of row r's token (position seq_lens[s] - q_len_s + r).  NULL
 *     k_new/v_new: the pool already holds every row's token.
 *   workspace : at least gw_attn_workspace_bytes(...) bytes (NULL when that
 *     is 0), 256-byte aligned, ZERO-FILLED before its first use; every call
 *     that completes leaves it ready for the next call of the same shape (it
 *     holds split counters that the call's last workgroups reset, and
 *     per-sequence call epochs).  Where those sit depends on the shape
 *     (num_seqs, KV and q heads, num_rows, max_q_len, max_seq_len, window):
 *     zero-fill it again before a call of another shape.  Calls that overlap
 *     in time must not share a workspace.
 *
 * Results are deterministic, and each row's result depends only on that
 * row's query, its sequence's length and K/V, the window and the scale --
 * not on the other rows of the call, their order, or where pages sit.
 */
size_t gw_attn_workspace_bytes(int32_t family, int32_t num_seqs, int32_t num_rows,
                               int32_t num_q_heads, int32_t head_dim, int32_t max_seq_len,
                               int32_t window, int32_t max_q_len);

/* Local family (pool->family == GW_FAMILY_LOCAL; bf16 or e4m3).
 * num_q_heads a multiple of num_kv_heads, group size 1, 2 or 4; window >= 1.
 * k_new / v_new: bf16 [num_rows][num_kv_heads][256]; with rot_dim 256 the
 * rotary tables (fp32 [max_pos][128]) are required, with rot_dim 0 they must
 * be NULL. */
int gw_decode_attn_local(const gw_pool_desc* pool /* host */, const void* q,
                         int32_t num_q_heads, const void* k_new, const void* v_new,
                         const float* rope_cos, const float* rope_sin, const int32_t* q_indptr,
                         const int32_t* seq_lens, const int32_t* page_table, int32_t pt_stride,
                         int32_t num_seqs, int32_t num_rows, int32_t max_q_len,
                         int32_t max_seq_len, int32_t window, float scale, float* out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* gw_decode_attn_local without a workspace argument, for callers that
 * cannot allocate device memory around the call (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, arithmetic, kernels and results as gw_decode_attn_local; the
 * split partials, counters and call epochs live instead in a scratch array
 * of the library's own, 32 MiB per GPU (static device memory, held until the
 * process ends).  A call whose plan needs more (gw_attn_workspace_bytes of
 * its shape above 32 MiB) returns GW_ERR_WORKSPACE before any HIP call.
 * Each call first clears the region it uses, so calls of any shape may
 * follow one another.  Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (concurrent streams or threads) race and
 * must be serialised by the caller.  The library allocates nothing here; the
 * array's device address is looked up once per device on the first call. */
int gw_decode_attn_local_noalloc(const gw_pool_desc* pool /* host */, const void* q,
                                 int32_t num_q_heads, const void* k_new, const void* v_new,
                                 const float* rope_cos, const float* rope_sin, const int32_t* q_indptr,
                                 const int32_t* seq_lens, const int32_t* page_table, int32_t pt_stride,
                                 int32_t num_seqs, int32_t num_rows, int32_t max_q_len,
                                 int32_t max_seq_len, int32_t window, float scale, float* out,
                                 void* stream);

/* Global family (GW_FAMILY_GLOBAL_COMPRESSED or GW_FAMILY_GLOBAL_FULL, bf16
 * or e4m3).  num_q_heads 16 or 32.  The two layouts give bit-identical
 * results.  An e4m3 pool is read as the exact bf16 values of its codes, for
 * decode and prompt rows alike; the rows' tokens appended in the call are
 * stored as the codes gw_kv_append stores.
 * v_new: bf16 [num_rows][512], with the rotary tables fp32 [max_pos][64];
 * NULL when the pool already holds the rows.  k_new: bf16 [num_rows][512],
 * each row's K before rotation, of which only dims 0..127 are read (the
 * quarter that rotates into K_rot), as gw_kv_append reads k_raw; NULL when K
 * is V before rotation (the tied store); set only with v_new. */
int gw_decode_attn_global(const gw_pool_desc* pool /* host */, const void* q,
                          int32_t num_q_heads, const void* k_new, const void* v_new, const float* rope_cos,
                          const float* rope_sin, const int32_t* q_indptr,
                          const int32_t* seq_lens, const int32_t* page_table, int32_t pt_stride,
                          int32_t num_seqs, int32_t num_rows, int32_t max_q_len,
                          int32_t max_seq_len, float scale, float* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------- pool lifecycle -- */
/*
 * Host page allocator of the two families (pegainfer "Gemma 4" page,
 * Scheduling): one object owns the page ids of one local and one global
 * pool (the same ids serve every layer of a family) and the decode slots.
 *   - Admission: a request of total_tokens (prompt + max_tokens) that will
 *     have at most max_step_rows query rows in one step is admitted into a
 *     free slot when both families' budgets hold its worst case: global,
 *     ceil(total / 16) pages (global pages are never freed while it runs);
 *     local, min(ceil(total / 16), (max_step_rows + window + 13) / 16 + 1)
 *     pages (the pages one step's rows and their windows can span).
 *     Otherwise it waits (*slot = -1, GW_OK) -- or, when no request is
 *     active and so nothing can free up, or total_tokens exceeds the
 *     ceiling max_context, it is refused (GW_ERR_REFUSED).
 *   - gw_alloc_extend: the slot's sequence now has new_len tokens and its
 *     earliest row still to be queried is at first_query_pos (new_len - 1
 *     for a decode step; non-decreasing; new_len - first_query_pos <=
 *     max_step_rows).  Pages are assigned to every logical page up to
 *     (new_len - 1) / 16 in both families; local pages wholly before
 *     first_query_pos - window + 1 go back to the free list, their table
 *     entries -1 (the attention kernels never read them).
 *   - gw_alloc_release: every page of the slot back, the slot free.
 *   - Free page ids are handed out lowest first, so the tables depend only
 *     on the sequence of calls.
 * All pointers here are host pointers; nothing touches the GPU.  One
 * allocator must not be called from two threads at once.
 */
typedef struct gw_page_alloc gw_page_alloc;

int gw_alloc_create(int32_t slots, int32_t max_context, int32_t window, int32_t local_pages,
                    int32_t global_pages, gw_page_alloc** out /* host */);
int gw_alloc_destroy(gw_page_alloc* a);
int gw_alloc_admit(gw_page_alloc* a, int32_t total_tokens, int32_t max_step_rows,
                   int32_t* slot /* host */);
int gw_alloc_extend(gw_page_alloc* a, int32_t slot, int32_t new_len, int32_t first_query_pos);
int gw_alloc_release(gw_page_alloc* a, int32_t slot);
/* Page tables as the attention calls take them (host int32, copied out):
 * local_pt [slots][local_stride], global_pt [slots][global_stride], both
 * strides >= ceil(max_context / 16), -1 where no page is held; seq_lens
 * [slots] (0 for a free slot) may be NULL. */
int gw_alloc_tables(const gw_page_alloc* a, int32_t* local_pt, int32_t local_stride, int32_t* global_pt,
                    int32_t global_stride, int32_t* seq_lens);
/* stats[6] (host): free local pages, free global pages, reserved local,
 * reserved global, active requests, slots. */
int gw_alloc_stats(const gw_page_alloc* a, int32_t* stats);

/*
 * Copy whole pages between two pools of the same family, dtype and
 * geometry: page dst_pages[i] of dst <- page src_pages[i] of src, i < n
 * (device int32 arrays).  This is the copy of the conversation prefix cache
 * (pegainfer "Gemma 4" page, Conversation prefix cache: finished prompt
 * states kept in pages of their own and copied back on a hit).  A pair with
 * an id outside its pool's [0, num_pages) is skipped.  Pairs must not write
 * the same destination page, nor read a page another pair writes.
 */
int gw_copy_pages(const gw_pool_desc* dst /* host */, const gw_pool_desc* src /* host */,
                  const int32_t* dst_pages, const int32_t* src_pages, int32_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GW_H */
