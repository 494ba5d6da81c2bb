// Global-family paged decode attention: head dim 512, one KV head shared by
// all q heads (MQA), K and V tied, K rebuilt from the compressed record.
//
// What is computed (pegainfer "Gemma 4" page, intro and Architecture notes;
// Gewell post, "the Why"): for each decode row at position p = seq_len - 1
// and each q head h, softmax over all keys j <= p of scale * q_h . K_j,
// applied to V_j, where K_j = [K_rot_j (dims 0..127) | V_j[128:512]] for the
// compressed record and K_j is read from its own block for the full record.
// Both records take the same arithmetic, so their results are bit-identical.
//
// With every q head on one KV head the score and value steps are dense
// contractions, so both run on MFMA (v_mfma_f32_16x16x32_bf16, fp32
// accumulation), in 16 x 16 blocks over a pair of pages (32 tokens):
//   S^T (16 tokens x 16 heads) = K (16 x 512) . Q^T (512 x 16 heads)
//                                  -- per page of the pair
//   O^T (16 dims x 16 heads)  += V^T (16 dims x 32 tokens) . P^T (32 x 16)
//                                  -- per 16-dim block, both pages at once
// The S^T results already sit in the lanes as the P^T operand wants them
// (lane l: head l % 16, tokens 4(l/16) .. +3 of each page; those eight
// tokens are the lane's k slots of the PV product), so the softmax of a pair
// stays in the wave, and the V^T operand holds the same eight tokens: the
// gfx950 transposing LDS reads give a lane one dim of four (bf16,
// ds_read_b64_tr_b16, once per page) or eight (e4m3, ds_read_b64_tr_b8, both
// pages in one read) tokens.
//
// Work split: one workgroup per (sequence, split) item, numbered compactly
// (workgroup b takes item b); a split is a balanced run of the row's pages
// (gw_plan.h), streamed in pairs straight from HBM into an LDS ring
// (global_load_lds_dwordx4, issued by the waves with time to spare).
// The score and value steps of a pair are split between waves and
// pipelined a pair apart (global_decode_ws_kernel: four score waves, each
// taking one page and half the score contraction's dims for every head, so
// each K fragment is read from LDS once, and four value waves, each taking
// 128 output dims of every head, so each V fragment is read once); the full
// bf16 record, whose 64 KiB pairs leave room for a ring of two only, runs
// both steps on all eight waves in turn (global_decode_full_kernel).  The
// partial scores of a page are added through LDS in a fixed order, scaled
// into the base-2 domain by the wave that computed them, and every wave that
// runs the softmax of a head holds the same scores and the same state, so
// all records take the same arithmetic and give bit-identical results.
// The running max moves only when a score passes it by more than 2^8 (the
// accumulators are rarely rescaled; the unnormalised weights stay below
// 2^8).  On the split's last pair, tokens past the row's position (and the
// missing second page of an odd split) get masked scores and zeroed V
// operands, so unwritten slots (possibly NaN) never reach the output.  P is
// rounded to bf16 for PV and the sum l adds exactly those rounded values
// (v_dot2_f32_bf16 against ones).  A row with several splits leaves each
// split's (acc, m, l) in the workspace, in MFMA fragment order, for
// global_split_reduce_kernel.

#include "gw_device.h"
#include "gw_kernels.h"
#include "gw_plan.h"
#include "gw_rows_append.h"

namespace gw {
namespace {

constexpr int kGD = 512;

// LDS ring depth: page slots of the wave-specialised kernel for the bf16
// compressed record (7 x 20 KiB), e4m3 compressed (8 x 10 KiB) and e4m3
// full (8 x 16 KiB), and pair slots of the full bf16 record's kernel
// (2 x 64 KiB); with the score exchange, one workgroup per CU.
#ifndef GW_GLOBAL_NS_C
#define GW_GLOBAL_NS_C 7
#endif
#ifndef GW_GLOBAL_NP_F
#define GW_GLOBAL_NP_F 2
#endif
#ifndef GW_GLOBAL_NS_C8
#define GW_GLOBAL_NS_C8 8
#endif
#ifndef GW_GLOBAL_NS_F8
#define GW_GLOBAL_NS_F8 8
#endif

// The reference max moves only when a score (base 2) passes it by more than this.
constexpr float kLazyMaxG = 8.f;
// bf16 1.0 in both halves: dot2_bf16(p, kBf16Ones, l) adds a pair of weights to l.
constexpr uint32_t kBf16Ones = 0x3f803f80u;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// FP8: the e4m3 page, its blocks in 16-dim chunks (16 bytes of a token).
template <bool COMPRESSED, bool FP8 = false>
struct GlobalPage {
  static constexpr int kBlock = FP8 ? 8192 : 16384;      // one [16][512] block
  static constexpr int kBytes = (COMPRESSED ? 5 : 8) * kBlock / 4;
  static constexpr int kVOff = COMPRESSED ? 0 : kBlock;  // V block inside the page
  // byte offset of dims 8c .. 8c+7 of token t of K inside the page
  __device__ static __forceinline__ int k_off(int c, int t) {
    const int kb = COMPRESSED && c < 16 ? kBlock : 0;   // compressed: dims < 128 from K_rot
    if constexpr (FP8) return kb + ((c >> 1) * 16 + t) * 16 + 8 * (c & 1);
    else return kb + (c * 16 + t) * 16;
  }
};

// Byte offset, inside a page, of what lane (g, l16) names in the transposing
// read of bf16 V for dims d_lo .. (lane (g, e, q) names token 4g + e, dims
// d_lo + 4q .. +3, and receives dim d_lo + l16 of tokens 4g .. 4g+3).
template <bool COMPRESSED>
__device__ __forceinline__ int global_v_lane_off(int d_lo, int g, int l16) {
  const int t_rd = 4 * g + (l16 >> 2);
  const int dd = d_lo + 4 * (l16 & 3);
  return GlobalPage<COMPRESSED>::kVOff + ((dd >> 3) * 16 + t_rd) * 16 + (dd & 7) * 2;
}

// 8 e4m3 codes -> 8 bf16 (exact), in order.
__device__ __forceinline__ bf16x8 widen_e4m3x8(uint32_t w0, uint32_t w1) {
  return __builtin_bit_cast(bf16x8, uint4{e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0),
                                          e4m3x2_to_bf16x2<false>(w1), e4m3x2_to_bf16x2<true>(w1)});
}

// The V^T operand of output block b (16 dims) for a pair of pages in LDS
// (page a at pa, page b at pb; for an e4m3 pair each lane's offset vo
// already names its page, as one transposing read spans both): lane (g, l16) gets dim (its
// block's first dim + l16) of tokens 4g .. 4g+3 of page a, then of page b,
// as 8 bf16.  vo: the lane's byte offset for block 0 (bf16:
// global_v_lane_off in a page; e4m3: the tr8 row it names, in page a or b).
template <bool COMPRESSED, bool FP8>
__device__ __forceinline__ uint4 global_pair_vt(const lds_u8* pa, const lds_u8* pb, int vo, int b) {
  if constexpr (FP8) {
    const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(pa + vo + 256 * b));
    return __builtin_bit_cast(uint4, widen_e4m3x8((uint32_t)r[0], (uint32_t)r[1]));
  } else {
    const uint2 va = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(pa + vo + 512 * b)));
    const uint2 vb = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(pb + vo + 512 * b)));
    return uint4{va.x, va.y, vb.x, vb.y};
  }
}

// s_waitcnt vmcnt(n) for a run-time n in 0 .. 31 (larger n waits for 31).
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  switch (n) {
#define GW_VMCNT_CASE(N) \
  case N: wait_vmcnt<N>(); break;
    GW_VMCNT_CASE(0) GW_VMCNT_CASE(1) GW_VMCNT_CASE(2) GW_VMCNT_CASE(3) GW_VMCNT_CASE(4) GW_VMCNT_CASE(5)
    GW_VMCNT_CASE(6) GW_VMCNT_CASE(7) GW_VMCNT_CASE(8) GW_VMCNT_CASE(9) GW_VMCNT_CASE(10) GW_VMCNT_CASE(11)
    GW_VMCNT_CASE(12) GW_VMCNT_CASE(13) GW_VMCNT_CASE(14) GW_VMCNT_CASE(15) GW_VMCNT_CASE(16) GW_VMCNT_CASE(17)
    GW_VMCNT_CASE(18) GW_VMCNT_CASE(19) GW_VMCNT_CASE(20) GW_VMCNT_CASE(21) GW_VMCNT_CASE(22) GW_VMCNT_CASE(23)
    GW_VMCNT_CASE(24) GW_VMCNT_CASE(25) GW_VMCNT_CASE(26) GW_VMCNT_CASE(27) GW_VMCNT_CASE(28) GW_VMCNT_CASE(29)
    GW_VMCNT_CASE(30)
#undef GW_VMCNT_CASE
    default: wait_vmcnt<31>(); break;
  }
}

// The (sequence, split) item of workgroup b: the call's items are numbered
// sequence by sequence (a decode row's splits in order), and workgroup b
// takes item b, so the active workgroups are 0 .. items-1 and spread evenly
// over the XCDs.  False past the last item.  Every value is wave-uniform.
struct GlobalItem {
  int s, split, nsplit, row, p;
};
__device__ __forceinline__ bool global_item(const GlobalAttnArgs& a, int b, int lane, GlobalItem& it) {
  int base = 0;
  for (int c = 0; c < a.num_seqs; c += 64) {
    const int sl = c + lane;
    int cnt = 0, len = 1, r0 = sl;
    if (sl < a.num_seqs) {
      len = a.seq_lens[sl];
      if (a.q_indptr) r0 = a.q_indptr[sl];
      if (!a.q_indptr || a.q_indptr[sl + 1] - r0 == 1) cnt = global_nsplit(((len - 1) >> 4) + 1);
    }
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int up = __shfl_up(incl, d, 64);
      incl += lane >= d ? up : 0;
    }
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (b < base + total) {
      const uint64_t hit = __ballot(base + incl > b);
      const int ls = __builtin_ctzll(hit);
      it.s = uniform_i32(c + ls);
      it.nsplit = uniform_i32(__builtin_amdgcn_readlane(cnt, ls));
      it.p = uniform_i32(__builtin_amdgcn_readlane(len, ls)) - 1;
      it.row = uniform_i32(__builtin_amdgcn_readlane(r0, ls));
      it.split = uniform_i32(b - (base + __builtin_amdgcn_readlane(incl, ls) - it.nsplit));
      return true;
    }
    base += total;
  }
  return false;
}

// A split's physical page ids (at most 256), 64 per register, read back
// with readlane so that the page loop issues no vector memory operation the
// compiler would wait on.
struct SplitPages {
  int v0, v1, v2, v3;
  __device__ __forceinline__ void load(const int32_t* pt, int n, int lane) {
    v0 = lane < n ? pt[lane] : 0;
    v1 = n > 64 && 64 + lane < n ? pt[64 + lane] : 0;
    v2 = n > 128 && 128 + lane < n ? pt[128 + lane] : 0;
    v3 = n > 192 && 192 + lane < n ? pt[192 + lane] : 0;
  }
  __device__ __forceinline__ int operator()(int i) const {
    const int l = i & 63;
    return i < 64 ? __builtin_amdgcn_readlane(v0, l)
         : i < 128 ? __builtin_amdgcn_readlane(v1, l)
         : i < 192 ? __builtin_amdgcn_readlane(v2, l)
                   : __builtin_amdgcn_readlane(v3, l);
  }
};


// ---------------------------------------------------------------------------
// Wave-specialised decode, for rings of three pairs or more (the compressed
// record and both e4m3 records): the score and the value steps of the pages
// run on separate waves and overlap, a pair apart.
//
//   score waves 0..3: wave w takes page w % 2 of the pair and dims
//     256 (w / 2) .. +255 of the score contraction, for every q head (its Q^T
//     operands stay in registers), so each K fragment is read from LDS once
//     and feeds the products of all head blocks; it leaves its partial
//     S^T blocks in an exchange buffer.
//   value waves 4..7: wave 4 + v adds the two partial sums of each score (in
//     a fixed order), runs the online softmax of every head (each value wave
//     holds the same full scores and keeps the same softmax state) and
//     accumulates O^T for dims 128 v .. +127 of every head, so each V
//     fragment is read once and feeds all head blocks.
//
// Step i of the loop: the score waves take pair i, the value waves pair
// i - 1 (exchange buffers alternate between steps), one barrier between
// steps.  The LDS ring holds NS pages (not pairs, so an odd count uses the
// space a pair ring would leave): the pages that slots freed by pair i - 2
// take are issued at step i, so NS - 4 pages are in flight while pairs i
// and i - 1 are read; q waits in the ring's last slots until the score
// waves have read it.
template <bool COMPRESSED, bool FP8, int HB>
__device__ __forceinline__ void global_tile_scores(f32x4 (&s)[HB], const lds_u8* pg, const bf16x8 (&qf)[HB][8],
                                                   int dh, int g, int l16) {
  using PG = GlobalPage<COMPRESSED, FP8>;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) s[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (FP8) {
    i32x2 kr[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) kr[k] = *reinterpret_cast<const lds_i32x2*>(pg + PG::k_off(4 * (8 * dh + k) + g, l16));
    __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the products
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const bf16x8 kf = widen_e4m3x8((uint32_t)kr[k][0], (uint32_t)kr[k][1]);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) s[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[hb][k], s[hb], 0, 0, 0);
    }
  } else {
    typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
    bf16x8 kf[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) kf[k] = *reinterpret_cast<const lds_bf16x8*>(pg + PG::k_off(4 * (8 * dh + k) + g, l16));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) s[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[k], qf[hb][k], s[hb], 0, 0, 0);
  }
}

template <bool COMPRESSED, int HB, int NS, bool FP8>
__global__ __launch_bounds__(512, 1) void global_decode_ws_kernel(GlobalAttnArgs a) {
  using PG = GlobalPage<COMPRESSED, FP8>;
  constexpr int kU = PG::kBytes / 1024;       // 1 KiB transfer units per page
  // page slot stride: e4m3 slots are 128 bytes apart beyond the page, so the
  // two pages a transposing V read spans (a pair sits in adjacent slots) hit
  // opposite halves of the 64 LDS banks; the pages' sizes are multiples of
  // the 256-byte bank width
  constexpr int kSlot = PG::kBytes + (FP8 ? 128 : 0);
  constexpr int kQPages = (HB * 16 * 1024 + kSlot - 1) / kSlot;   // page slots q holds at first
  constexpr int kXsBytes = HB * 4 * 1024;     // one pair's partial scores: [page][dim half][hb][lane] f32x4
  constexpr int kXsOff = NS * kSlot;
  // pages issued before the loop: every slot q does not hold, at most 10
  // (so that no wait below counts more than 31 transfers of a score wave),
  // and at least pairs 0 and 1: step 1 waits for pair 1 before it issues
  constexpr int kPro = NS - kQPages < 10 ? NS - kQPages : 10;
  static_assert(NS >= 6 && kPro >= 4 && (NS - 4) * ((kU + 3) / 4) <= 31 && kPro * ((kU + 3) / 4) <= 31, "ring depth");
  static_assert(!FP8 || NS % 2 == 0, "an e4m3 pair's pages sit side by side");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kXsOff + 2 * kXsBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = uniform_i32(tid >> 6);
  const bool scorer = w < 4;
  // trace slots: 0 XCD | split << 8 | sequence << 32, 1 pairs, 2 entry,
  // 3 pair 0 in LDS, 4 step 1 open, 5 value waves' loop done, 6 score
  // waves' loop done, 7 exit (value wave 4)
  GW_TRACE_T(a, 2, tid == 0);
  const int g = lane >> 4, l16 = lane & 15;
  // the workgroups past the decode items append the prompt rows' own
  // tokens, two units of 256 threads each (the prompt rows attend in a
  // later launch)
  if ((int)blockIdx.x >= a.append_wg0) {
    global_rows_append_unit<COMPRESSED, FP8>(a, ((int)blockIdx.x - a.append_wg0) * 2 + tid / 256, tid % 256);
    return;
  }

  GlobalItem it;
  if (!global_item(a, blockIdx.x, lane, it)) return;
  const int s = it.s, split = it.split, nsplit = it.nsplit, row = it.row, p = it.p;
  const int n_pages = (p >> 4) + 1;
  const int pg0 = split_lo(n_pages, nsplit, split);
  const int n = split_lo(n_pages, nsplit, split + 1) - pg0;
  const int n_pairs = (n + 1) >> 1;

  // ---- the split's page ids, waited for here: the compiler does not see
  // the direct-to-LDS transfers below, and a wait of its own placed after
  // them would hold for them too
  SplitPages phys;
  phys.load(a.page_table + (int64_t)s * a.pt_stride + pg0, n, lane);
  asm volatile("" ::"v"(phys.v0), "v"(phys.v1), "v"(phys.v2), "v"(phys.v3));
  // the decode row's own token, when the call carries it: on the workgroup
  // of the row's last split, value wave 7 (idle while the score waves take
  // pair 0) rotates it, stores it into the pool (as gw_kv_append does) and,
  // before that page's scores, into the page's LDS copy
  const bool append_here = a.v_new != nullptr && split == nsplit - 1;
  constexpr int kAppendWave = 7;
  GlobalRecordLane rec{};

  // ---- q into the ring's last kQPages slots (1 KiB per head, chunk c of
  // head h at chunk c ^ (h % 8), so the operand reads hit distinct banks),
  // ahead of the pages; wave w moves heads 2 HB w .. +2 HB - 1
  uint8_t* qs = smem + (NS - kQPages) * kSlot;
  {
    const uint32_t qs_lds = uniform_i32((int)lds_address(qs));
#pragma unroll
    for (int i = 0; i < 2 * HB; ++i) {
      const int h = 2 * HB * w + i;
      dma16_to_lds(a.q + ((int64_t)row * a.num_q_heads + h) * kGD + 8 * (lane ^ (h & 7)),
                   qs_lds + (uint32_t)(h * 1024));
    }
  }

  // ---- transfers: page q of the split (pages 2j, 2j + 1 make pair j; an
  // odd split's last pair repeats its last page as the second, whose scores
  // are masked and V zeroed) lands in page slot q % NS, in the pool's
  // layout; its 1 KiB unit u is moved by score wave (kU q + u) % 4.  The
  // value waves, the pipeline's longer path, issue no page transfers: a
  // direct-to-LDS transfer can hold its wave at issue for a good part of a
  // microsecond when many are in flight, and that stall then falls on the
  // waves with time to spare.  The waits count page transfers only: q's
  // transfers are older than all of them, and the appending wave (a value
  // wave) has no page transfers, so each of its waits covers its pool stores.
  const uint32_t ring_lds = uniform_i32((int)lds_address(smem));
  const int n_pg = 2 * n_pairs;
  auto first_unit = [&](int q) __attribute__((always_inline)) { return (w - kU * q) & 3; };
  auto units_of = [&](int q) __attribute__((always_inline)) {
    if (!scorer) return 0;
    const int u0 = first_unit(q);
    return u0 < kU ? (kU - 1 - u0) / 4 + 1 : 0;
  };
  auto issue_page = [&](int q) __attribute__((always_inline)) {
    if (!scorer) return;
    const uint8_t* src = a.pool + (int64_t)phys(min(q, n - 1)) * a.page_bytes + 16 * lane;
    const uint32_t dst = ring_lds + (uint32_t)((q % NS) * kSlot);
    const int u0 = first_unit(q);
#pragma unroll
    for (int k = 0; k < (kU + 3) / 4; ++k) {
      const int u = u0 + 4 * k;
      if (u < kU) dma16_to_lds(src + 1024 * u, dst + 1024 * u);
    }
  };
  // pages 0 .. last landed: this wave's transfers of the later pages issued
  // so far may stay in flight
  int issued = min(kPro, n_pg);   // pages issued so far (uniform)
  auto wait_through = [&](int last) __attribute__((always_inline)) {
    int after = 0;
    for (int q = last + 1; q < issued; ++q) after += units_of(q);
    wait_vmcnt_upto(after);
  };
  for (int q = 0; q < issued; ++q) issue_page(q);
  auto page_lds = [&](int q) __attribute__((always_inline)) {
    return (const lds_u8*)(uintptr_t)(ring_lds + (uint32_t)((q % NS) * kSlot));
  };

  // ---- the loop's synchronisation, the same on both roles: step i > 0
  // opens with pair i in LDS (this wave's transfers, then the barrier), pair
  // i - 1's partial scores in, pair i - 2 done, and issues the pages whose
  // slots that freed; the appending workgroup patches the split's last page
  // before its scores
  f32x4* xs = reinterpret_cast<f32x4*>(smem + kXsOff);
  auto step_open = [&](int i) __attribute__((always_inline)) {
    if (i > 0) {
      if (i < n_pairs) wait_through(2 * i + 1);
      lds_barrier();
      const int lim = min(2 * i - 3 + NS, n_pg - 1);
      while (issued <= lim) issue_page(issued++);
    }
    if (append_here && i == n_pairs - 1) {
      if (w == kAppendWave)
        put_global_record_as<COMPRESSED, FP8>(smem + ((n - 1) % NS) * kSlot, rec, p & 15, lane);
      lds_barrier();
    }
  };
  // pair 0 and q in LDS for every wave
  wait_through(1);
  lds_barrier();
  GW_TRACE_T(a, 3, tid == 0);
  GW_TRACE_V(a, 0, tid == 0, GW_TRACE_XCC() | (uint64_t)split << 8 | (uint64_t)s << 32);
  GW_TRACE_V(a, 1, tid == 0, n_pairs);

  if (scorer) {
    // ---- score waves: Q^T operands (head 16 hb + l16, dims 256 dh + 32 k +
    // 8g .. +7) from LDS once, then per step the page's partial S^T blocks
    const int t_sc = w & 1, dh = w >> 1;
    bf16x8 qf[HB][8];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int h = 16 * hb + l16, c = 4 * (8 * dh + k) + g;
        qf[hb][k] = *reinterpret_cast<const bf16x8*>(qs + h * 1024 + ((c ^ (h & 7)) * 16));
      }
    for (int i = 0; i <= n_pairs; ++i) {
      step_open(i);
      if (i < n_pairs) {
        f32x4 sc[HB];
        global_tile_scores<COMPRESSED, FP8, HB>(
            sc, page_lds(2 * i + t_sc), qf, dh, g, l16);
        f32x4* xb = xs + (i & 1) * (kXsBytes / 16);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) xb[((2 * t_sc + dh) * HB + hb) * 64 + lane] = sc[hb] * a.scale_log2;
      }
    }
    GW_TRACE_T(a, 6, tid == 0);
    return;
  }

  // ---- value waves: output dims v_lo .. +127 of every head
  if (append_here && w == kAppendWave) {
    rec = global_record_lane(a.v_new + (int64_t)row * kGD, (a.k_new ? a.k_new : a.v_new) + (int64_t)row * kGD,
                             a.rope_cos, a.rope_sin, p, lane);
    put_global_record_as<COMPRESSED, FP8>(const_cast<uint8_t*>(a.pool) + (int64_t)phys(n - 1) * a.page_bytes, rec,
                                          p & 15, lane);
  }
  const int v_lo = 128 * (w - 4);
  f32x4 acc[HB][8];
  float m_run[HB], l_run[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    m_run[hb] = -INFINITY;
    l_run[hb] = 0.f;
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[hb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // V^T read offset of block 0 (bf16: the tr16 lane offset inside page a,
  // page b at + kBytes; e4m3: the tr8 row r = l16 / 2 names token 4g + r % 4
  // of page a (r < 4) or b, half l16 % 2 of the block's 16 dims)
  int vo;
  if constexpr (FP8) {
    const int r = l16 >> 1;
    vo = (r < 4 ? 0 : kSlot) + PG::kVOff + (((v_lo >> 4) * 16 + 4 * g + (r & 3)) * 16) + 8 * (l16 & 1);
  } else {
    vo = global_v_lane_off<COMPRESSED>(v_lo, g, l16);
  }
  for (int i = 0; i <= n_pairs; ++i) {
    step_open(i);
    GW_TRACE_T(a, 4, tid == 256 && i == 1);
    if (i == 0) continue;
    {
      const int j = i - 1;
      const lds_u8* pa = page_lds(2 * j);
      const lds_u8* pbp = page_lds(2 * j + 1);
      uint4 vf[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) vf[b] = global_pair_vt<COMPRESSED, FP8>(pa, pbp, vo, b);
      const f32x4* xb = xs + (j & 1) * (kXsBytes / 16);
      // lane: head 16 hb + l16, tokens 4g .. 4g+3 of page a (t = 0) and b
      float z[HB][2][4];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const f32x4 sc = xb[((2 * t + 0) * HB + hb) * 64 + lane] + xb[((2 * t + 1) * HB + hb) * 64 + lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) z[hb][t][r] = sc[r];
        }
      // the split's last pair: tokens past p and a missing second page masked
      const bool last = j == n_pairs - 1;   // uniform
      uint32_t vm[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
      if (last) {
        const int tok_a = (pg0 + 2 * j) * 16 + 4 * g;
        const bool b_ok = 2 * j + 1 < n;
        bool ok[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) ok[t][r] = tok_a + 16 * t + r <= p && (t == 0 || b_ok);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) z[hb][t][r] = ok[t][r] ? z[hb][t][r] : -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            vm[2 * t + h] = (ok[t][2 * h] ? 0x0000ffffu : 0u) | (ok[t][2 * h + 1] ? 0xffff0000u : 0u);
      }
      float mx[HB];
      bool grow = false;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        mx[hb] = max_lanes_xor16_32(fmaxf(fmaxf(fmaxf(z[hb][0][0], z[hb][0][1]), fmaxf(z[hb][0][2], z[hb][0][3])),
                                          fmaxf(fmaxf(z[hb][1][0], z[hb][1][1]), fmaxf(z[hb][1][2], z[hb][1][3]))));
        grow = grow || mx[hb] > m_run[hb] + kLazyMaxG;
      }
      if (__any(grow)) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const bool up = mx[hb] > m_run[hb] + kLazyMaxG;
          const float alpha = up ? __builtin_amdgcn_exp2f(m_run[hb] - mx[hb]) : 1.f;
#pragma unroll
          for (int b = 0; b < 8; ++b) acc[hb][b] *= alpha;
          l_run[hb] *= alpha;
          m_run[hb] = up ? mx[hb] : m_run[hb];
        }
      }
      bf16x8 pb[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        uint32_t pp[4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            pp[2 * t + h] = pack_bf16(__builtin_amdgcn_exp2f(z[hb][t][2 * h] - m_run[hb]),
                                      __builtin_amdgcn_exp2f(z[hb][t][2 * h + 1] - m_run[hb]));
        l_run[hb] = dot2_bf16(pp[3], kBf16Ones, dot2_bf16(pp[2], kBf16Ones,
                              dot2_bf16(pp[1], kBf16Ones, dot2_bf16(pp[0], kBf16Ones, l_run[hb]))));
        pb[hb] = __builtin_bit_cast(bf16x8, uint4{pp[0], pp[1], pp[2], pp[3]});
      }
      if (last) {
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          vf[b].x &= vm[0];
          vf[b].y &= vm[1];
          vf[b].z &= vm[2];
          vf[b].w &= vm[3];
        }
      }
#pragma unroll
      for (int b = 0; b < 8; ++b)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
          acc[hb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf[b]), pb[hb], acc[hb][b], 0,
                                                               0, 0);
    }
  }

  GW_TRACE_T(a, 5, tid == 256);
  // ---- write: lane holds head 16 hb + l16, dims v_lo + 16b + 4g .. +3
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = 16 * hb + l16;
    const float l_tot = sum_lanes_xor16_32(l_run[hb]);
    if (nsplit == 1) {
      float* op = a.out + ((int64_t)row * a.num_q_heads + head) * kGD + v_lo + 4 * g;
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int b = 0; b < 8; ++b) *reinterpret_cast<f32x4*>(op + 16 * b) = acc[hb][b] * inv;
    } else {
      const int64_t item = (int64_t)s * a.max_splits + split;
      f32x4* op = reinterpret_cast<f32x4*>(a.part_acc) + ((item * HB + hb) * 32 + (v_lo >> 4)) * 64 + lane;
#pragma unroll
      for (int b = 0; b < 8; ++b) op[64 * b] = acc[hb][b];
      if (v_lo == 0 && g == 0) {
        a.part_ml[(item * a.num_q_heads + head) * 2 + 0] = m_run[hb];
        a.part_ml[(item * a.num_q_heads + head) * 2 + 1] = l_tot;
      }
    }
  }
  GW_TRACE_T(a, 7, tid == 256);
}

// The full bf16 record (64 KiB pairs, a ring of two): all eight waves on
// every pair, scores first, then softmax and PV.  The arithmetic is that of
// global_decode_ws_kernel step for step, so both records give bit-identical
// results: wave w computes the S^T block of page (w / 2) % 2, dim half w / 4
// and head block w % 2 (with 16 heads: page w % 2, half w / 2, waves 0..3),
// the partial sums are added in the same order, and wave w then takes head
// block w % 2 and output dims 128 (w / 2) .. +127 (16 heads: dims 64 w ..
// +63) of the softmax and PV steps.
template <int HB, int NP>
__global__ __launch_bounds__(512, 1) void global_decode_full_kernel(GlobalAttnArgs a) {
  using PG = GlobalPage<false>;
  constexpr int kPair = 2 * PG::kBytes;
  constexpr int kUnits = kPair / 1024;        // 1 KiB transfer units per pair (8 per wave)
  constexpr int kPerWave = kUnits / 8;
  constexpr int kBlocks = HB == 2 ? 8 : 4;    // 16-dim output blocks per wave
  constexpr int kXsOff = NP * kPair;          // partial scores: [page][dim half][hb][lane] f32x4
  static_assert(kUnits % 8 == 0 && NP >= 2 && kPerWave * (NP - 2) < 64 && NP - 2 <= 4, "ring depth");
  static_assert(kPair >= HB * 16 * 1024, "a ring slot holds q");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kXsOff + HB * 4 * 1024];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = uniform_i32(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  // trace slots: those of global_decode_ws_kernel, 3 q in LDS, 5 loop done
  GW_TRACE_T(a, 2, tid == 0);
  const bool scorer = HB == 2 || w < 4;
  const int t_sc = HB == 2 ? (w >> 1) & 1 : w & 1;     // score block: page,
  const int dh = HB == 2 ? w >> 2 : (w >> 1) & 1;      // dim half,
  const int hb = HB == 2 ? w & 1 : 0;                   // head block (also of the PV step)
  const int d_lo = HB == 2 ? 128 * (w >> 1) : 64 * w;   // output dims d_lo .. + 16 kBlocks
  // the workgroups past the decode items append the prompt rows' own tokens
  if ((int)blockIdx.x >= a.append_wg0) {
    global_rows_append_unit<false, false>(a, ((int)blockIdx.x - a.append_wg0) * 2 + tid / 256, tid % 256);
    return;
  }

  GlobalItem it;
  if (!global_item(a, blockIdx.x, lane, it)) return;
  const int s = it.s, split = it.split, nsplit = it.nsplit, row = it.row, p = it.p;
  const int n_pages = (p >> 4) + 1;
  const int pg0 = split_lo(n_pages, nsplit, split);
  const int n = split_lo(n_pages, nsplit, split + 1) - pg0;
  const int n_pairs = (n + 1) >> 1;
  const int head = 16 * hb + l16;

  // ---- the split's physical page ids and, on the wave that appends a
  // decode row's own token, that token's inputs go out first, in one round
  // trip, and are waited for before anything else is issued: the compiler
  // does not see the direct-to-LDS transfers below, and a wait of its own
  // placed after them would hold for them too.  The workgroup of the row's
  // last split rotates the token and stores it into the pool (as
  // gw_kv_append does) before any transfer, and into its LDS copy of that
  // page once the page has landed.
  SplitPages phys;
  phys.load(a.page_table + (int64_t)s * a.pt_stride + pg0, n, lane);
  const bool append_here = a.v_new != nullptr && split == nsplit - 1;
  GlobalRecordLane rec{};
  if (append_here && w == 0)
    rec = global_record_lane(a.v_new + (int64_t)row * kGD, (a.k_new ? a.k_new : a.v_new) + (int64_t)row * kGD,
                             a.rope_cos, a.rope_sin, p, lane);
  asm volatile("" ::"v"(phys.v0), "v"(phys.v1), "v"(phys.v2), "v"(phys.v3));
  if (append_here && w == 0)
    put_global_record<false>(const_cast<uint8_t*>(a.pool) + (int64_t)phys(n - 1) * a.page_bytes, rec, p & 15, lane);

  // ---- q into ring slot NP - 1 (free until the loop's first transfer) by
  // direct transfers: 1 KiB per head, the row's 16-byte chunk c of head h at
  // chunk c ^ (h % 8), so that the Q^T operand reads hit distinct banks
  uint8_t* qs = smem + (NP - 1) * kPair;
  {
    const uint32_t qs_lds = uniform_i32((int)lds_address(qs));
#pragma unroll
    for (int i = 0; i < 2 * HB; ++i) {
      const int h = 2 * HB * w + i;
      dma16_to_lds(a.q + ((int64_t)row * a.num_q_heads + h) * kGD + 8 * (lane ^ (h & 7)),
                   qs_lds + (uint32_t)(h * 1024));
    }
  }

  // ---- transfers: unit u (1 KiB) of pair j is unit u % (kUnits / 2) of
  // page 2j (u < kUnits / 2) or page 2j + 1, landing at unit u of the pair's
  // ring slot (the pool's layout); wave w moves units kPerWave w .. +kPerWave
  // - 1.  An odd split's last pair repeats its last page as the second; that
  // copy's scores are masked and its V zeroed.
  const uint32_t ring_lds = uniform_i32((int)lds_address(smem));
  auto issue_pair = [&](int j) __attribute__((always_inline)) {
    const uint8_t* src0 = a.pool + (int64_t)phys(2 * j) * a.page_bytes + 16 * lane;
    const uint8_t* src1 = a.pool + (int64_t)phys(min(2 * j + 1, n - 1)) * a.page_bytes + 16 * lane;
    const uint32_t dst = ring_lds + (uint32_t)((j % NP) * kPair);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int u = kPerWave * w + i;
      constexpr int kHalf = kUnits / 2;
      dma16_to_lds(u < kHalf ? src0 + 1024 * u : src1 + 1024 * (u - kHalf), dst + 1024 * u);
    }
  };
#pragma unroll
  for (int j = 0; j < NP - 1; ++j)
    if (j < n_pairs) issue_pair(j);

  // Q^T operands of the wave's score block (head 16 hb + l16, dims 256 dh +
  // 32 k + 8g .. +7), once every wave's q transfers are in
  wait_groups_after<kPerWave>(min(NP - 1, n_pairs));
  lds_barrier();
  GW_TRACE_T(a, 3, tid == 0);
  GW_TRACE_V(a, 0, tid == 0, GW_TRACE_XCC() | (uint64_t)split << 8 | (uint64_t)s << 32);
  GW_TRACE_V(a, 1, tid == 0, n_pairs);
  bf16x8 qf[1][8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = 4 * (8 * dh + k) + g;
    qf[0][k] = *reinterpret_cast<const bf16x8*>(qs + head * 1024 + ((c ^ (head & 7)) * 16));
  }
  f32x4* xs = reinterpret_cast<f32x4*>(smem + kXsOff);

  f32x4 acc[kBlocks];
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int vo = global_v_lane_off<false>(d_lo, g, l16);

  for (int j = 0; j < n_pairs; ++j) {
    wait_groups_after<kPerWave>(min(NP - 2, n_pairs - 1 - j));
    lds_barrier();   // pair j is in LDS for every wave; pair j - 1 is done
    if (j + NP - 1 < n_pairs) issue_pair(j + NP - 1);
    const lds_u8* pa = (const lds_u8*)(uintptr_t)(ring_lds + (uint32_t)((j % NP) * kPair));
    if (append_here && j == n_pairs - 1) {
      if (w == 0) put_global_record<false>(smem + (j % NP) * kPair + ((n - 1) & 1) * PG::kBytes, rec, p & 15, lane);
      lds_barrier();
    }
    if (scorer) {
      f32x4 sc[1];
      global_tile_scores<false, false, 1>(sc, pa + t_sc * PG::kBytes, qf, dh, g, l16);
      xs[((2 * t_sc + dh) * HB + hb) * 64 + lane] = sc[0] * a.scale_log2;
    }
    lds_barrier();

    // ---- online softmax for head l16 over the pair's 32 tokens (lane:
    // tokens 4g .. 4g+3 of page a, then of page b); on the split's last
    // pair, tokens past p and a missing second page are masked
    float z[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f32x4 sc = xs[((2 * t + 0) * HB + hb) * 64 + lane] + xs[((2 * t + 1) * HB + hb) * 64 + lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) z[t][r] = sc[r];
    }
    const bool last = j == n_pairs - 1;   // uniform
    uint32_t vm[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
    if (last) {
      const int tok_a = (pg0 + 2 * j) * 16 + 4 * g;
      const bool b_ok = 2 * j + 1 < n;
      bool ok[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ok[t][r] = tok_a + 16 * t + r <= p && (t == 0 || b_ok);
          z[t][r] = ok[t][r] ? z[t][r] : -INFINITY;
        }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          vm[2 * t + h] = (ok[t][2 * h] ? 0x0000ffffu : 0u) | (ok[t][2 * h + 1] ? 0xffff0000u : 0u);
    }
    const float mx = max_lanes_xor16_32(fmaxf(fmaxf(fmaxf(z[0][0], z[0][1]), fmaxf(z[0][2], z[0][3])),
                                              fmaxf(fmaxf(z[1][0], z[1][1]), fmaxf(z[1][2], z[1][3]))));
    if (__any(mx > m_run + kLazyMaxG)) {
      const bool up = mx > m_run + kLazyMaxG;
      const float alpha = up ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
#pragma unroll
      for (int b = 0; b < kBlocks; ++b) acc[b] *= alpha;
      l_run *= alpha;
      m_run = up ? mx : m_run;
    }
    uint32_t pp[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        pp[2 * t + h] = pack_bf16(__builtin_amdgcn_exp2f(z[t][2 * h] - m_run), __builtin_amdgcn_exp2f(z[t][2 * h + 1] - m_run));
    l_run = dot2_bf16(pp[3], kBf16Ones, dot2_bf16(pp[2], kBf16Ones, dot2_bf16(pp[1], kBf16Ones, dot2_bf16(pp[0], kBf16Ones, l_run))));
    const bf16x8 pb = __builtin_bit_cast(bf16x8, uint4{pp[0], pp[1], pp[2], pp[3]});

    // ---- O^T += V^T . P^T over the pair's 32 tokens, per 16-dim block
    uint4 vf[kBlocks];
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) vf[b] = global_pair_vt<false, false>(pa, pa + PG::kBytes, vo, b);
    if (last) {
#pragma unroll
      for (int b = 0; b < kBlocks; ++b) {
        vf[b].x &= vm[0];
        vf[b].y &= vm[1];
        vf[b].z &= vm[2];
        vf[b].w &= vm[3];
      }
    }
#pragma unroll
    for (int b = 0; b < kBlocks; ++b)
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf[b]), pb, acc[b], 0, 0, 0);
  }

  GW_TRACE_T(a, 5, tid == 0);
  // ---- write: lane holds head 16hb + l16, dims d_lo + 16b + 4g .. +3
  const float l_tot = sum_lanes_xor16_32(l_run);
  if (nsplit == 1) {
    float* op = a.out + ((int64_t)row * a.num_q_heads + head) * kGD + d_lo + 4 * g;
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) *reinterpret_cast<f32x4*>(op + 16 * b) = acc[b] * inv;
  } else {
    const int64_t item = (int64_t)s * a.max_splits + split;
    f32x4* op = reinterpret_cast<f32x4*>(a.part_acc) + ((item * HB + hb) * 32 + (d_lo >> 4)) * 64 + lane;
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) op[64 * b] = acc[b];
    if (d_lo == 0 && g == 0) {
      a.part_ml[(item * a.num_q_heads + head) * 2 + 0] = m_run;
      a.part_ml[(item * a.num_q_heads + head) * 2 + 1] = l_tot;
    }
  }
  GW_TRACE_T(a, 7, tid == 0);
}

// The scores half of the page for the prompt rows: S^T = K . Q^T per row
// (16 steps over 512 dims, two accumulation chains, K read in batches of 4
// fragments).
template <bool COMPRESSED, bool FP8, int NR>
__device__ __forceinline__ void global_rows_scores(f32x4 (&s)[NR][2], const uint8_t* pg, const bf16x8 (&qf)[NR][16],
                                                   int g, int l16) {
  using PG = GlobalPage<COMPRESSED, FP8>;
#pragma unroll
  for (int r = 0; r < NR; ++r) s[r][0] = s[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int hk = 0; hk < 4; ++hk) {
    bf16x8 kf[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (FP8) {   // e4m3 codes widen to bf16 exactly
        const i32x2 kr = *reinterpret_cast<const i32x2*>(pg + PG::k_off(4 * (4 * hk + k) + g, l16));
        kf[k] = widen_e4m3x8((uint32_t)kr[0], (uint32_t)kr[1]);
      } else {
        kf[k] = *reinterpret_cast<const bf16x8*>(pg + PG::k_off(4 * (4 * hk + k) + g, l16));
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int r = 0; r < NR; ++r)
        s[r][k & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[k], qf[r][4 * hk + k], s[r][k & 1], 0, 0, 0);
  }
}

// One page for the prompt rows: a wave takes one head block (16 heads) of NR
// rows over all 512 dims, so no wave repeats another's scores and each K
// and V fragment it reads from LDS feeds NR rows' products.  Per page:
// the scores (global_rows_scores, issued a page ahead), the lazy
// online-softmax update per row, then O^T += V^T . P^T over 32 output
// blocks of 16 dims (V read in batches of 4 blocks; an e4m3 page's
// transposing read gives the operands of two blocks, widened exactly).  V
// of tokens past p_v (slots past the workgroup's last row, possibly never
// written) is zeroed in the operand registers.
template <bool COMPRESSED, bool FP8, int NR>
__device__ __forceinline__ void global_rows_page(f32x4 (&acc)[NR][32], float (&m_run)[NR], float (&l_run)[NR],
                                                 const uint8_t* pg, const f32x4 (&s)[NR][2], int tok_page0,
                                                 const int (&p)[NR], int p_v, int g, int l16, int v_lane_off,
                                                 float scale_log2) {
  const int tok0 = tok_page0 + 4 * g;
  s16x4 pb[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const f32x4 sacc = s[r][0] + s[r][1];
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = (tok0 + i <= p[r]) ? sacc[i] * scale_log2 : -INFINITY;
    const float mx = max_lanes_xor16_32(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
    // the reference max moves only when a score passes it by more than 2^8
    if (__any(mx > m_run[r] + 8.f)) {
      const bool up = mx > m_run[r] + 8.f;
      const float alpha = up ? __builtin_amdgcn_exp2f(m_run[r] - mx) : 1.f;
#pragma unroll
      for (int b = 0; b < 32; ++b) acc[r][b] *= alpha;
      l_run[r] *= alpha;
      m_run[r] = up ? mx : m_run[r];
    }
    const uint32_t p01 = pack_bf16(__builtin_amdgcn_exp2f(z[0] - m_run[r]), __builtin_amdgcn_exp2f(z[1] - m_run[r]));
    const uint32_t p23 = pack_bf16(__builtin_amdgcn_exp2f(z[2] - m_run[r]), __builtin_amdgcn_exp2f(z[3] - m_run[r]));
    l_run[r] += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
    pb[r] = __builtin_bit_cast(s16x4, uint2{p01, p23});
  }
  const bool tail = tok_page0 + 15 > p_v;   // uniform
  uint32_t vm0 = 0xffffffffu, vm1 = 0xffffffffu;
  if (tail) {
    vm0 = (tok0 + 0 <= p_v ? 0x0000ffffu : 0u) | (tok0 + 1 <= p_v ? 0xffff0000u : 0u);
    vm1 = (tok0 + 2 <= p_v ? 0x0000ffffu : 0u) | (tok0 + 3 <= p_v ? 0xffff0000u : 0u);
  }
  lds_u8* vrow = (lds_u8*)pg + v_lane_off;
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) {
    uint2 vf[4];
    if constexpr (FP8) {   // blocks 2j, 2j + 1 per read, 512 bytes per pair of 16-dim chunks
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vrow + 512 * (2 * bb + h)));
        vf[2 * h] = uint2{e4m3x2_to_bf16x2<false>((uint32_t)r[0]), e4m3x2_to_bf16x2<true>((uint32_t)r[0])};
        vf[2 * h + 1] = uint2{e4m3x2_to_bf16x2<false>((uint32_t)r[1]), e4m3x2_to_bf16x2<true>((uint32_t)r[1])};
      }
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b)
        vf[b] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vrow + 512 * (4 * bb + b))));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      uint2 vv = vf[b];
      vv.x &= vm0;
      vv.y &= vm1;
#pragma unroll
      for (int r = 0; r < NR; ++r)
        acc[r][4 * bb + b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vv), pb[r],
                                                                       acc[r][4 * bb + b], 0, 0, 0);
    }
  }
}

// Cross-split reduce: M = max_i m_i, l = sum_i l_i 2^(m_i - M),
// out = sum_i acc_i 2^(m_i - M) / l.  The partials sit in MFMA fragment
// order (fragment (hb, block) of a split: 64 lanes x 4 floats, lane
// g*16 + l16 holding head 16 hb + l16, dims 16 block + 4g .. +3), so every
// load moves 1 KiB in one piece.  The order of the additions depends on the
// row's split count only: the splits go in chunks of kReduceChunk, each
// chunk's state (its max, and l and acc relative to it, summed in split
// order) is computed on its own in one round trip, and the chunk states are
// folded in chunk order.  Two ways to schedule the same arithmetic:
//   sequential: a wave per fragment folds its chunks one after another
//     (four fragments per unit of 256 threads);
//   parallel: the four waves of a unit take chunks 4r .. 4r + 3 of one
//     fragment at once and the first folds them, round r after round r - 1
//     (rows of many splits: C3's 64 splits in one round trip).
constexpr int kReduceChunk = 16;
constexpr int kReduceWaves = 4;
// LDS of a parallel unit: the round's chunk states, [wave][m, l, acc x 4][lane]
constexpr int kReduceLdsFloats = kReduceWaves * 6 * 64;

struct ReduceState {
  float m, l;
  f32x4 o;
};

// State of splits [c0, c0 + nc) of the fragment (pa, ml: the lane's split-0 records).
__device__ __forceinline__ ReduceState reduce_chunk(const f32x4* pa, const float* ml, int64_t acc_step,
                                                    int64_t ml_step, int c0, int nc) {
  f32x4 v[kReduceChunk];
  float2 x[kReduceChunk];
#pragma unroll
  for (int i = 0; i < kReduceChunk; ++i) {
    v[i] = i < nc ? pa[(c0 + i) * acc_step] : f32x4{0.f, 0.f, 0.f, 0.f};
    x[i] = i < nc ? *reinterpret_cast<const float2*>(ml + (c0 + i) * ml_step) : float2{-INFINITY, 0.f};
  }
  ReduceState st{-INFINITY, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int i = 0; i < kReduceChunk; ++i) st.m = fmaxf(st.m, x[i].x);
#pragma unroll
  for (int i = 0; i < kReduceChunk; ++i) {
    if (i < nc) {
      const float w = __builtin_amdgcn_exp2f(x[i].x - st.m);
      st.l += x[i].y * w;
      st.o += v[i] * w;
    }
  }
  return st;
}

// acc <- acc folded with the next chunk's state c (an empty state, max
// -inf, adds nothing; the first fold returns c exactly).
__device__ __forceinline__ void reduce_fold(ReduceState& acc, const ReduceState& c) {
  const float mn = fmaxf(acc.m, c.m);
  const float wa = acc.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(acc.m - mn);
  const float wc = c.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(c.m - mn);
  acc.l = acc.l * wa + c.l * wc;
  acc.o = acc.o * wa + c.o * wc;
  acc.m = mn;
}

// The row and split count of decode sequence s (false: not a decode row,
// or one split, written by the decode kernel itself).
__device__ __forceinline__ bool reduce_row(const ReduceArgs& a, int s, int& row, int& nsplit) {
  row = s;
  if (a.q_indptr) {
    row = a.q_indptr[s];
    if (a.q_indptr[s + 1] - row != 1) return false;
  }
  nsplit = global_nsplit(cdiv_i(a.seq_lens[s], kPage));
  return nsplit > 1;
}

__device__ __forceinline__ void reduce_store(const ReduceArgs& a, int row, int frag, int lane, const ReduceState& st) {
  const int head = 16 * (frag >> 5) + (lane & 15);
  *reinterpret_cast<f32x4*>(a.out + ((int64_t)row * a.num_q_heads + head) * kGD + 16 * (frag & 31) + 4 * (lane >> 4)) =
      st.o / st.l;
}

// Sequential schedule: sequence s, fragments 4y .. 4y + 3, by 256 threads
// (tid 0 .. 255), one wave per fragment.
__device__ __forceinline__ void global_split_reduce_unit(const ReduceArgs& a, int s, int y, int tid) {
  const int lane = tid & 63;
  const int frag = y * 4 + (tid >> 6);   // hb * 32 + block
  const int hbs = a.num_q_heads / 16;
  if (frag >= hbs * 32) return;
  int row, nsplit;
  if (!reduce_row(a, s, row, nsplit)) return;
  const int head = 16 * (frag >> 5) + (lane & 15);
  const f32x4* pa = reinterpret_cast<const f32x4*>(a.part_acc) + ((int64_t)s * a.max_splits * hbs * 32 + frag) * 64 + lane;
  const float* ml = a.part_ml + ((int64_t)s * a.max_splits * a.num_q_heads + head) * 2;
  const int64_t acc_step = (int64_t)hbs * 32 * 64, ml_step = 2 * (int64_t)a.num_q_heads;
  ReduceState st{-INFINITY, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
  for (int c0 = 0; c0 < nsplit; c0 += kReduceChunk)
    reduce_fold(st, reduce_chunk(pa, ml, acc_step, ml_step, c0, min(kReduceChunk, nsplit - c0)));
  reduce_store(a, row, frag, lane, st);
}

// Parallel schedule: sequence s (blockIdx.x), fragment blockIdx.y.
__global__ __launch_bounds__(256) void global_split_reduce_par_kernel(ReduceArgs a) {
  __shared__ float red[kReduceLdsFloats];
  const int s = blockIdx.x, frag = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, k = tid >> 6;
  int row, nsplit;
  if (!reduce_row(a, s, row, nsplit)) return;   // uniform over the workgroup
  const int hbs = a.num_q_heads / 16;
  const int head = 16 * (frag >> 5) + (lane & 15);
  const f32x4* pa = reinterpret_cast<const f32x4*>(a.part_acc) + ((int64_t)s * a.max_splits * hbs * 32 + frag) * 64 + lane;
  const float* ml = a.part_ml + ((int64_t)s * a.max_splits * a.num_q_heads + head) * 2;
  const int64_t acc_step = (int64_t)hbs * 32 * 64, ml_step = 2 * (int64_t)a.num_q_heads;
  const int nchunk = cdiv_i(nsplit, kReduceChunk);
  ReduceState st{-INFINITY, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
  for (int r0 = 0; r0 < nchunk; r0 += kReduceWaves) {
    const int c = r0 + k;
    const ReduceState cs = c < nchunk ? reduce_chunk(pa, ml, acc_step, ml_step, c * kReduceChunk,
                                                     min(kReduceChunk, nsplit - c * kReduceChunk))
                                      : ReduceState{-INFINITY, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
    float* q = red + k * 6 * 64 + lane;
    q[0] = cs.m;
    q[64] = cs.l;
    q[128] = cs.o[0];
    q[192] = cs.o[1];
    q[256] = cs.o[2];
    q[320] = cs.o[3];
    __syncthreads();
    if (k == 0) {
      for (int j = 0; j < kReduceWaves && r0 + j < nchunk; ++j) {
        const float* qj = red + j * 6 * 64 + lane;
        reduce_fold(st, ReduceState{qj[0], qj[64], f32x4{qj[128], qj[192], qj[256], qj[320]}});
      }
    }
    __syncthreads();
  }
  if (k == 0) reduce_store(a, row, frag, lane, st);
}

__global__ __launch_bounds__(256) void global_split_reduce_kernel(ReduceArgs a) {
  global_split_reduce_unit(a, blockIdx.x, blockIdx.y, threadIdx.x);
}


// Prompt rows (sequences with more than one query row: a new prompt's
// rows, or a chunk of one after a cached prefix, computed in the same step
// as the decode rows -- pegainfer "Gemma 4" page, Scheduling).  Row r of
// sequence s sits at position p_r = seq_len - q_len + r and attends keys
// 0 .. p_r.  kW = 8 / NR waves; wave (hb, rp) takes head block hb of rows
// NR rp .. NR rp + NR - 1 of the workgroup's kW NR / HB rows (NR = 1: two
// waves per SIMD; two rows per wave do not fit the registers), through a
// ring of NS pages that all waves fill.  No split: a row's whole range is
// one pass, and the output is written directly.  Items are (prompt
// sequence, row group), numbered compactly level by level (every
// sequence's last group first, then every sequence's second last, ...: the
// longest ranges of the call first).
template <bool COMPRESSED, bool FP8, int HB, int NR, int NS>
__global__ __launch_bounds__(64 * (8 / NR), 1) void global_prefill_kernel(GlobalAttnArgs a) {
  using PG = GlobalPage<COMPRESSED, FP8>;
  constexpr int kW = 8 / NR;                  // waves
  constexpr int kUnits = PG::kBytes / 1024;
  constexpr int kPerWave = kUnits / kW;       // units per wave per page ...
  constexpr int kPerWaveTail = kUnits % kW;   // ... the first kUnits % kW waves one more
  constexpr int kRows = kW * NR / HB;         // rows per workgroup
  static_assert(NR != 1 || kRows == global_prefill_rows(16 * HB), "the host's item count");
  // NS >= 3: iteration i reads page i + 1, issued an iteration earlier
  static_assert(NS >= 3 && NS - 2 <= 4 && (kPerWave + 1) * (NS - 2) < 64, "ring depth");
  __shared__ __attribute__((aligned(16))) uint8_t ring[NS][PG::kBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  // trace slots (row kTracePrefillRow + b): 0 XCD | row group << 8 |
  // sequence << 32, 1 pages, 2 entry, 3 first page in LDS, 4 wave 0's loop
  // done, 5 iteration 1 open, 6 last iteration open, 7 exit, 8 + w wave w's
  // loop done
  const int trow = kTracePrefillRow + (int)blockIdx.x;
  GW_TRACE_AT(a, trow, 2, tid == 0);
  // the first reduce_wgs workgroups merge the decode rows' splits (the
  // decode kernel, an earlier launch, wrote them), two units of 256 threads
  // each; placed ahead of the prompt-row items, their short work folds into
  // the items' schedule instead of trailing it
  if ((int)blockIdx.x < a.reduce_wgs) {
    const int u = (int)blockIdx.x * 2 + tid / 256;
    const int groups = reduce_groups(a.num_q_heads);
    if (u < a.num_seqs * groups) {
      const ReduceArgs r{a.q_indptr, a.seq_lens, a.part_acc, a.part_ml, a.out, a.num_q_heads, a.max_splits};
      global_split_reduce_unit(r, u / groups, u % groups, tid % 256);
    }
    return;
  }
  const int wv = uniform_i32(tid >> 6);
  const int hb = HB == 2 ? (wv & 1) : 0;
  const int rp = HB == 2 ? (wv >> 1) : wv;
  const int g = lane >> 4, l16 = lane & 15;
  const int head = 16 * hb + l16;

  int s = -1, mg = 0, row0 = 0, q_len = 0, L = 0;
  {
    PromptItem it;
    if (prompt_item(a.q_indptr, a.seq_lens, a.num_seqs, kRows, (int)blockIdx.x - a.reduce_wgs, lane, it)) {
      s = it.s;
      mg = it.grp;
      row0 = it.row0;
      q_len = it.q_len;
      L = it.len;
    }
  }
  if (s < 0) return;
  s = uniform_i32(s);
  mg = uniform_i32(mg);
  row0 = uniform_i32(row0);
  q_len = uniform_i32(q_len);
  L = uniform_i32(L);

  // the workgroup's rows kRows mg .. r_last; this wave's rows compute on
  // r_last's query and position when they lie past it (and are not written)
  const int r_last = min(kRows * mg + kRows - 1, q_len - 1);
  const int p_last = L - q_len + r_last;
  const int n = (p_last >> 4) + 1;
  GW_TRACE_VAT(a, trow, 0, tid == 0, GW_TRACE_XCC() | (uint64_t)mg << 8 | (uint64_t)s << 32);
  GW_TRACE_VAT(a, trow, 1, tid == 0, n);
  int rw[NR], pr[NR];
  bool rok[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    rw[i] = kRows * mg + NR * rp + i;
    rok[i] = rw[i] <= r_last;
    pr[i] = L - q_len + (rok[i] ? rw[i] : r_last);
  }

  // wave wv moves units [u0, u0 + nu) of every page
  const int nu = kPerWave + (wv < kPerWaveTail ? 1 : 0);
  const int u0 = kPerWave * wv + min(wv, kPerWaveTail);
  PageIds ids;
  ids.init(a.page_table + (int64_t)s * a.pt_stride, n, lane);
  const uint32_t ring_base = uniform_i32((int)lds_address(&ring[0][0])) + (uint32_t)(1024 * u0);
  auto issue_page = [&](int i) __attribute__((always_inline)) {
    const uint8_t* src = a.pool + (int64_t)ids.get(i) * a.page_bytes + 1024 * u0 + 16 * lane;
    const uint32_t dst = ring_base + (uint32_t)((i % NS) * PG::kBytes);
#pragma unroll
    for (int u = 0; u < kPerWave + 1; ++u)
      if (u < nu) dma16_to_lds(src + 1024 * u, dst + 1024 * u);
  };
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (i < n) issue_page(i);

  bf16x8 qf[NR][16];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const uint16_t* qp = a.q + ((int64_t)(row0 + (rok[i] ? rw[i] : r_last)) * a.num_q_heads + head) * kGD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[i][ks] = __builtin_bit_cast(bf16x8, ld16_cached(qp + 32 * ks));
  }

  f32x4 acc[NR][32];
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int b = 0; b < 32; ++b) acc[i][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NR], l_run[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }
  // V^T read offset of block 0 (bf16: the tr16 lane offset; e4m3: the tr8
  // row r = l16 / 2 names token 4g + r % 4 of 16-dim chunk r / 4 (blocks 0
  // and 1), half l16 % 2 of its 16 dims)
  const int v_lane_off = FP8 ? PG::kVOff + ((((l16 >> 1) >> 2) * 16 + 4 * g + ((l16 >> 1) & 3)) * 16) + 8 * (l16 & 1)
                             : global_v_lane_off<COMPRESSED>(0, g, l16);

  // software pipeline, one page deep: iteration i has pages i and i + 1 in
  // LDS; page i + 1's scores go out beside page i's weights and products
  if (nu > kPerWave) wait_groups_after<kPerWave + 1>(min(NS - 2, n - 1));
  else wait_groups_after<kPerWave>(min(NS - 2, n - 1));
  lds_barrier();
  GW_TRACE_AT(a, trow, 3, tid == 0);
  f32x4 sc[NR][2];
  global_rows_scores<COMPRESSED, FP8, NR>(sc, ring[0], qf, g, l16);
  for (int i = 0; i < n; ++i) {
    if (nu > kPerWave) wait_groups_after<kPerWave + 1>(max(0, min(NS - 3, n - 2 - i)));
    else wait_groups_after<kPerWave>(max(0, min(NS - 3, n - 2 - i)));
    lds_barrier();   // pages i and i + 1 are in LDS for every wave; page i - 1 is done
    GW_TRACE_AT(a, trow, 5, tid == 0 && i == 1);
    GW_TRACE_AT(a, trow, 6, tid == 0 && i == n - 1);
    if (i + NS - 1 < n) issue_page(i + NS - 1);
    f32x4 sn[NR][2];
    global_rows_scores<COMPRESSED, FP8, NR>(sn, ring[min(i + 1, n - 1) % NS], qf, g, l16);
    global_rows_page<COMPRESSED, FP8, NR>(acc, m_run, l_run, ring[i % NS], sc, i * 16, pr, p_last, g, l16, v_lane_off,
                                     a.scale_log2);
#pragma unroll
    for (int r = 0; r < NR; ++r) { sc[r][0] = sn[r][0]; sc[r][1] = sn[r][1]; }
  }
  GW_TRACE_AT(a, trow, 4, tid == 0);
  GW_TRACE_AT(a, trow, 8 + wv, lane == 0);
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if (!rok[i]) continue;
    const float inv = 1.f / sum_lanes_xor16_32(l_run[i]);
    float* op = a.out + ((int64_t)(row0 + rw[i]) * a.num_q_heads + head) * kGD + 4 * g;
    // streaming stores (written back now rather than evicted later during a
    // decode kernel's stream)
#pragma unroll
    for (int b = 0; b < 32; ++b) __builtin_nontemporal_store(acc[i][b] * inv, reinterpret_cast<f32x4*>(op + 16 * b));
  }
  GW_TRACE_AT(a, trow, 7, tid == 0);
}

}  // namespace

hipError_t launch_split_reduce(const ReduceArgs& a, int num_seqs, hipStream_t stream) {
  // rows of more than two chunks of splits take the parallel schedule (the
  // same arithmetic: the choice moves no result)
  if (a.max_splits > 2 * kReduceChunk) {
    dim3 grid(num_seqs, a.num_q_heads / 16 * 32), block(256);
    hipLaunchKernelGGL(global_split_reduce_par_kernel, grid, block, 0, stream, a);
  } else {
    dim3 grid(num_seqs, reduce_groups(a.num_q_heads)), block(256);
    hipLaunchKernelGGL(global_split_reduce_kernel, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_global_decode(const GlobalAttnArgs& a_in, bool compressed, bool fp8, hipStream_t stream) {
  // the decode items, then the prompt rows' append units (two per workgroup)
  const int64_t n_dec = (int64_t)a_in.max_splits * a_in.num_seqs;
  const int64_t n = n_dec + (a_in.append_units + 1) / 2;
  if (n > 0x7fffffff) return hipErrorInvalidConfiguration;
  GlobalAttnArgs a = a_in;
  a.append_wg0 = (int32_t)n_dec;
  dim3 grid((unsigned)n), block(512);
  const bool h32 = a.num_q_heads == 32;
  constexpr int kNc = GW_GLOBAL_NS_C, kNf = GW_GLOBAL_NP_F, kNc8 = GW_GLOBAL_NS_C8, kNf8 = GW_GLOBAL_NS_F8;
  if (fp8) {
    if (compressed) {
      if (h32) hipLaunchKernelGGL((global_decode_ws_kernel<true, 2, kNc8, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((global_decode_ws_kernel<true, 1, kNc8, true>), grid, block, 0, stream, a);
    } else {
      if (h32) hipLaunchKernelGGL((global_decode_ws_kernel<false, 2, kNf8, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((global_decode_ws_kernel<false, 1, kNf8, true>), grid, block, 0, stream, a);
    }
  } else if (compressed) {
    if (h32) hipLaunchKernelGGL((global_decode_ws_kernel<true, 2, kNc, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((global_decode_ws_kernel<true, 1, kNc, false>), grid, block, 0, stream, a);
  } else {
    if (h32) hipLaunchKernelGGL((global_decode_full_kernel<2, kNf>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((global_decode_full_kernel<1, kNf>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_global_prefill(const GlobalAttnArgs& a_in, bool compressed, bool fp8, int max_q_len,
                                 hipStream_t stream) {
  // the decode rows' cross-split reduce (two units of 256 threads per
  // workgroup) when the decode rows have splits, then one workgroup per
  // (prompt sequence, group of 8 / HB rows) (the entry point has checked
  // that the count fits a grid)
  const bool h32 = a_in.num_q_heads == 32;
  const long long items =
      prefill_items(a_in.num_rows, a_in.num_seqs, max_q_len, global_prefill_rows(a_in.num_q_heads));
  const long long n_red =
      a_in.max_splits > 1 ? ((long long)a_in.num_seqs * reduce_groups(a_in.num_q_heads) + 1) / 2 : 0;
  if (items + n_red == 0) return hipSuccess;
  if (items + n_red > 0x7fffffff) return hipErrorInvalidConfiguration;
  GlobalAttnArgs a = a_in;
  a.reduce_wgs = (int32_t)n_red;
  dim3 grid((unsigned)(items + n_red)), block(512);
#define GW_GPREFILL_CASE(C_, F_)                                                                      \
  if (compressed == C_ && fp8 == F_) {                                                                \
    if (h32) hipLaunchKernelGGL((global_prefill_kernel<C_, F_, 2, 1, 3>), grid, block, 0, stream, a); \
    else hipLaunchKernelGGL((global_prefill_kernel<C_, F_, 1, 1, 3>), grid, block, 0, stream, a);     \
    return hipGetLastError();                                                                         \
  }
  GW_GPREFILL_CASE(true, false) GW_GPREFILL_CASE(false, false) GW_GPREFILL_CASE(true, true)
  GW_GPREFILL_CASE(false, true)
#undef GW_GPREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace gw
