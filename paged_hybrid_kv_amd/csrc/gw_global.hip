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
// (gw_plan.h).  The split's pages go by in pairs, and all eight waves work on
// every pair: wave w takes head block hb (16 heads: w % 2 with 32 q heads,
// the only block with 16), 128 of the score contraction's 512 dims (part w / 2,
// or w % 4 with 16 heads) and a slice of the output dims (128 dims with 32
// heads, 64 with 16).  The waves of a head block add their partial scores
// through LDS in a fixed part order, so every wave of the block holds the same
// full scores and the same online-softmax state.  The running max moves only
// when a score passes it by more than 2^8 (so the accumulators are rarely
// rescaled; the unnormalised weights stay below 2^8).  Pages stream straight
// from HBM into a ring of LDS pair slots (global_load_lds_dwordx4, every wave
// moving its share of every pair), NP - 1 pairs in flight while one is read.
// On the split's last pair, tokens past the row's position (and the missing
// second page of an odd split) get masked scores and zeroed V operands, so
// unwritten slots (possibly NaN) never reach the output.  P is rounded to
// bf16 for PV and the sum l adds exactly those rounded values.

#include "gw_device.h"
#include "gw_kernels.h"
#include "gw_plan.h"

namespace gw {
namespace {

constexpr int kGD = 512;

// LDS ring depth in page pairs: bf16 compressed / full record (3 x 40 KiB,
// 2 x 64 KiB), e4m3 compressed / full (5 x 20 KiB, 3 x 32 KiB, q in a 32
// KiB region of its own); with the 16 KiB score exchange, one workgroup per CU.
#ifndef GW_GLOBAL_NP_C
#define GW_GLOBAL_NP_C 3
#endif
#ifndef GW_GLOBAL_NP_F
#define GW_GLOBAL_NP_F 2
#endif
#ifndef GW_GLOBAL_NP_C8
#define GW_GLOBAL_NP_C8 5
#endif
#ifndef GW_GLOBAL_NP_F8
#define GW_GLOBAL_NP_F8 3
#endif

// The reference max moves only when a score (base 2) passes it by more than this.
constexpr float kLazyMaxG = 8.f;

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

// A pair of pages in LDS (page a at pa, page b at pa + kBytes), for one wave:
//
// global_pair_scores: the wave's share of S^T = K . Q^T for both pages, over
// the four 32-dim steps 4 sp .. 4 sp + 3 of its score part (the waves of a
// head block add their shares through LDS); lane holds head l16, tokens
// 4g .. 4g+3 of each page.  All eight K fragments are read before the
// products.  e4m3 fragments (8 bytes) widen exactly to bf16 just before
// their product.
template <bool COMPRESSED, bool FP8>
__device__ __forceinline__ void global_pair_scores(f32x4 (&s)[2], const lds_u8* pa, const bf16x8 (&qf)[4], int sp,
                                                   int g, int l16) {
  using PG = GlobalPage<COMPRESSED, FP8>;
  if constexpr (FP8) {
    i32x2 kr[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        kr[t][k] = *reinterpret_cast<const lds_i32x2*>(pa + t * PG::kBytes + PG::k_off(4 * (4 * sp + k) + g, l16));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen_e4m3x8((uint32_t)kr[t][k][0], (uint32_t)kr[t][k][1]),
                                                       qf[k], s[t], 0, 0, 0);
    }
  } else {
    typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
    bf16x8 kf[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        kf[t][k] = *reinterpret_cast<const lds_bf16x8*>(pa + t * PG::kBytes + PG::k_off(4 * (4 * sp + k) + g, l16));
    __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the products
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 4; ++k) s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t][k], qf[k], s[t], 0, 0, 0);
    }
  }
}

// The V^T operand of output block b (16 dims) for the pair: lane (g, l16)
// gets dim (its block's first dim + l16) of tokens 4g .. 4g+3 of page a,
// then of page b, as 8 bf16.  vo: the lane's byte offset for block 0 (bf16:
// global_v_lane_off in page a; e4m3: the tr8 row it names, in page a or b).
template <bool COMPRESSED, bool FP8>
__device__ __forceinline__ uint4 global_pair_vt(const lds_u8* pa, int vo, int b) {
  if constexpr (FP8) {
    const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(pa + vo + 256 * b));
    return __builtin_bit_cast(uint4, widen_e4m3x8((uint32_t)r[0], (uint32_t)r[1]));
  } else {
    constexpr int kB = GlobalPage<COMPRESSED>::kBytes;
    const uint2 va = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(pa + vo + 512 * b)));
    const uint2 vb =
        __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(pa + kB + vo + 512 * b)));
    return uint4{va.x, va.y, vb.x, vb.y};
  }
}

// One workgroup = eight waves on one (sequence, split) item; see the header
// for the work split.  NP: page pairs in the LDS ring (NP - 1 pairs in
// flight while one is read).  FP8: e4m3 pages, widened to bf16 as they are
// read from LDS; q then has an LDS region of its own after the ring.
template <bool COMPRESSED, int HB, int NP, bool FP8 = false>
__global__ __launch_bounds__(512, 1) void global_decode_kernel(GlobalAttnArgs a) {
  using PG = GlobalPage<COMPRESSED, FP8>;
  constexpr int kPair = 2 * PG::kBytes;
  constexpr int kUnits = kPair / 1024;        // 1 KiB transfer units per pair
  constexpr int kEven = kUnits / 8;           // units every wave moves ...
  constexpr int kExtra = kUnits % 8;          // ... and one more for waves below kExtra
  constexpr int kPerWave = kEven + (kExtra > 0 ? 1 : 0);
  constexpr int kBlocks = HB == 2 ? 8 : 4;    // 16-dim output blocks per wave
  constexpr int kRingBytes = NP * kPair;
  constexpr int kXsOff = kRingBytes;          // score exchange: [wave][lane][page] f32x4
  constexpr int kQOff = kXsOff + 8 * 64 * 32; // e4m3: q
  static_assert(NP >= 2 && kPerWave * (NP - 2) < 64 && NP - 2 <= 4, "ring depth");
  static_assert(FP8 || kPair >= 32 * 1024, "a ring slot holds q");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kQOff + (FP8 ? 32 * 1024 : 0)];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = uniform_i32(tid >> 6);
  const int hb = HB == 2 ? (w & 1) : 0;
  const int sp = HB == 2 ? (w >> 1) : (w & 3);          // score part: dims 128 sp ..
  const int d_lo = HB == 2 ? 128 * (w >> 1) : 64 * w;   // output dims d_lo .. + 16 kBlocks
  const int g = lane >> 4, l16 = lane & 15;

  // ---- work item of this workgroup: the call's (sequence, split) items are
  // numbered sequence by sequence, and workgroup b takes item b, so the
  // active workgroups are 0 .. items-1 and spread evenly over the XCDs
  int s = -1, split = 0, nsplit = 1, L = 1, row = 0;
  {
    const int b = blockIdx.x;
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
        s = c + ls;
        nsplit = __builtin_amdgcn_readlane(cnt, ls);
        L = __builtin_amdgcn_readlane(len, ls);
        row = __builtin_amdgcn_readlane(r0, ls);
        split = b - (base + __builtin_amdgcn_readlane(incl, ls) - nsplit);
        break;
      }
      base += total;
    }
  }
  if (s < 0) return;
  s = uniform_i32(s);
  split = uniform_i32(split);
  nsplit = uniform_i32(nsplit);
  L = uniform_i32(L);
  row = uniform_i32(row);
  const int p = L - 1;
  const int n_pages = (p >> 4) + 1;
  const int pg0 = split_lo(n_pages, nsplit, split);
  const int n = split_lo(n_pages, nsplit, split + 1) - pg0;
  const int n_pairs = (n + 1) >> 1;
  const int head = 16 * hb + l16;

  // ---- the split's physical page ids (one per lane and register, read
  // back with readlane; a split has at most 256 pages) and, on the wave that
  // appends a decode row's own token, that token's inputs go out first, in
  // one round trip, and are waited for before anything else is issued: the
  // compiler does not see the direct-to-LDS transfers below, and a wait of
  // its own placed after them would hold for them too.
  const int32_t* pt = a.page_table + (int64_t)s * a.pt_stride + pg0;
  auto pt_at = [&](int idx) __attribute__((always_inline)) { return idx < n ? pt[idx] : 0; };
  const int ptv0 = pt_at(lane);
  const int ptv1 = n > 64 ? pt_at(64 + lane) : 0;
  const int ptv2 = n > 128 ? pt_at(128 + lane) : 0;
  const int ptv3 = n > 192 ? pt_at(192 + lane) : 0;
  auto phys = [&](int i) __attribute__((always_inline)) {
    const int l = i & 63;
    return i < 64 ? __builtin_amdgcn_readlane(ptv0, l)
         : i < 128 ? __builtin_amdgcn_readlane(ptv1, l)
         : i < 192 ? __builtin_amdgcn_readlane(ptv2, l)
                   : __builtin_amdgcn_readlane(ptv3, l);
  };
  // a decode row's own token, when the call carries it: the workgroup of the
  // row's last split rotates it and stores it into the pool (as
  // gw_kv_append does) before any transfer, and into its LDS copy of that
  // page once the page has landed
  const bool append_here = a.v_new != nullptr && split == nsplit - 1;
  GlobalRecordLane rec{};
  if (append_here && w == 0)
    rec = global_record_lane(a.v_new + (int64_t)row * kGD, a.v_new + (int64_t)row * kGD, a.rope_cos, a.rope_sin, p, lane);
  asm volatile("" ::"v"(ptv0), "v"(ptv1), "v"(ptv2), "v"(ptv3));
  if (append_here && w == 0)
    put_global_record_as<COMPRESSED, FP8>(const_cast<uint8_t*>(a.pool) + (int64_t)phys(n - 1) * a.page_bytes, rec,
                                          p & 15, lane);

  // ---- q into LDS by direct transfers, ahead of the pages (bf16: in ring
  // slot NP - 1, free until the loop's first transfer): 1 KiB per head, the
  // row's 16-byte chunk c of head h stored at chunk c ^ (h % 8), so that the
  // Q^T operand reads below hit distinct banks.  Wave w moves heads
  // 2 HB w .. +2 HB - 1; lane i fetches the chunk that lands at position i.
  uint8_t* qs = FP8 ? smem + kQOff : smem + (NP - 1) * kPair;
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
  // ring slot, so the LDS copy has the pool's layout.  Wave w moves units
  // kEven w .. + kEven - 1 and, below kExtra, unit 8 kEven + w.  An odd
  // split's last pair repeats its last page as the second; that copy's
  // scores are masked and its V zeroed.  The loop's waits count transfers
  // only; the appending wave's pool stores and the q transfers are older
  // than all of them, so they are covered too.
  const int my_units = kEven + (w < kExtra ? 1 : 0);
  const uint32_t ring_base = uniform_i32((int)lds_address(smem));
  auto issue_pair = [&](int j) __attribute__((always_inline)) {
    const uint8_t* src0 = a.pool + (int64_t)phys(2 * j) * a.page_bytes + 16 * lane;
    const uint8_t* src1 = a.pool + (int64_t)phys(min(2 * j + 1, n - 1)) * a.page_bytes + 16 * lane;
    const uint32_t dst = ring_base + (uint32_t)((j % NP) * kPair);
    auto unit = [&](int u) __attribute__((always_inline)) {
      constexpr int kHalf = kUnits / 2;
      const uint8_t* src = u < kHalf ? src0 + 1024 * u : src1 + 1024 * (u - kHalf);
      dma16_to_lds(src, dst + 1024 * u);
    };
#pragma unroll
    for (int u = 0; u < kEven; ++u) unit(kEven * w + u);
    if (kExtra > 0 && w < kExtra) unit(8 * kEven + w);
  };
  // at most k pairs' transfers of this wave left in flight
  auto wait_pairs_after = [&](int k) __attribute__((always_inline)) {
    if (kExtra > 0 && my_units == kEven) wait_groups_after<(kExtra > 0 ? kEven : kPerWave)>(k);
    else wait_groups_after<kPerWave>(k);
  };
#pragma unroll
  for (int j = 0; j < NP - 1; ++j)
    if (j < n_pairs) issue_pair(j);

  // Q^T operand for the wave's score part: head 16hb + l16, dims
  // 32 ks + 8g .. +7 (16-byte chunk 4ks + g), ks = 4 sp + k, once every
  // wave's q transfers (older than its page transfers) are in
  wait_pairs_after(min(NP - 1, n_pairs));
  lds_barrier();
  bf16x8 qf[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int ks = 4 * sp + k;
    qf[k] = *reinterpret_cast<const bf16x8*>(qs + head * 1024 + (((4 * ks + g) ^ (head & 7)) * 16));
  }
  f32x4* xs = reinterpret_cast<f32x4*>(smem + kXsOff);

  f32x4 acc[kBlocks];
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  // V^T read offsets: bf16, the tr16 lane offset inside page a (page b at
  // + kBytes); e4m3, the tr8 row r = l16 / 2 of the lane's group names token
  // 4g + r % 4 of page a (r < 4) or b, half l16 % 2 of the block's 16 dims
  int vo;
  if constexpr (FP8) {
    const int r = l16 >> 1;
    vo = (r < 4 ? 0 : PG::kBytes) + PG::kVOff + (((d_lo >> 4) * 16 + 4 * g + (r & 3)) * 16) + 8 * (l16 & 1);
  } else {
    vo = global_v_lane_off<COMPRESSED>(d_lo, g, l16);
  }
  const uint32_t ring_lds = uniform_i32((int)lds_address(smem));

  for (int j = 0; j < n_pairs; ++j) {
    wait_pairs_after(min(NP - 2, n_pairs - 1 - j));
    lds_barrier();   // pair j is in LDS for every wave; pair j - 1 is done
    if (j + NP - 1 < n_pairs) issue_pair(j + NP - 1);
    const uint32_t slot = ring_lds + (uint32_t)((j % NP) * kPair);
    const lds_u8* pa = (const lds_u8*)(uintptr_t)slot;
    if (append_here && j == ((n - 1) >> 1)) {
      if (w == 0) put_global_record_as<COMPRESSED, FP8>(smem + (j % NP) * kPair + ((n - 1) & 1) * PG::kBytes, rec,
                                                        p & 15, lane);
      lds_barrier();
    }
    // ---- scores: the wave's part, then the head block's four parts added
    // in part order
    f32x4 sc[2];
    global_pair_scores<COMPRESSED, FP8>(sc, pa, qf, sp, g, l16);
    if (HB == 2 || w < 4) {
      xs[(w * 64 + lane) * 2 + 0] = sc[0];
      xs[(w * 64 + lane) * 2 + 1] = sc[1];
    }
    lds_barrier();
    const int w0 = HB == 2 ? hb : 0, ws = HB == 2 ? 2 : 1;   // wave of part q: w0 + ws q
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f32x4 x0 = xs[((w0 + 0 * ws) * 64 + lane) * 2 + t], x1 = xs[((w0 + 1 * ws) * 64 + lane) * 2 + t];
      const f32x4 x2 = xs[((w0 + 2 * ws) * 64 + lane) * 2 + t], x3 = xs[((w0 + 3 * ws) * 64 + lane) * 2 + t];
      sc[t] = (x0 + x1) + (x2 + x3);
    }

    // ---- online softmax for head l16 over the pair's 32 tokens; on the
    // split's last pair, tokens past p and a missing second page are masked
    const int tok_a = (pg0 + 2 * j) * 16 + 4 * g;   // the lane's first token of page a; page b: + 16
    const bool last = j == n_pairs - 1;             // uniform
    float z[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) z[t][r] = sc[t][r] * a.scale_log2;
    uint32_t vm[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
    if (last) {
      const bool b_ok = 2 * j + 1 < n;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = tok_a + 16 * t + r <= p && (t == 0 || b_ok);
          z[t][r] = ok ? z[t][r] : -INFINITY;
        }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          vm[2 * t + h] = (z[t][2 * h] != -INFINITY ? 0x0000ffffu : 0u) | (z[t][2 * h + 1] != -INFINITY ? 0xffff0000u : 0u);
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
    l_run += ((bf16_lo(pp[0]) + bf16_hi(pp[0])) + (bf16_lo(pp[1]) + bf16_hi(pp[1]))) +
             ((bf16_lo(pp[2]) + bf16_hi(pp[2])) + (bf16_lo(pp[3]) + bf16_hi(pp[3])));
    const bf16x8 pb = __builtin_bit_cast(bf16x8, uint4{pp[0], pp[1], pp[2], pp[3]});

    // ---- O^T += V^T . P^T over the pair's 32 tokens, per 16-dim block
    uint4 vf[kBlocks];
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) vf[b] = global_pair_vt<COMPRESSED, FP8>(pa, vo, b);
    __builtin_amdgcn_sched_barrier(0);
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

  // ---- write: lane holds head 16hb + l16, dims d_lo + 16b + 4g .. +3
  const float l_tot = sum_lanes_xor16_32(l_run);
  if (nsplit == 1) {
    float* op = a.out + ((int64_t)row * a.num_q_heads + head) * kGD + d_lo + 4 * g;
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) *reinterpret_cast<f32x4*>(op + 16 * b) = acc[b] * inv;
  } else {
    const int64_t pi = ((int64_t)s * a.num_q_heads + head) * a.max_splits + split;
    float* op = a.part_acc + pi * kGD + d_lo + 4 * g;
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) *reinterpret_cast<f32x4*>(op + 16 * b) = acc[b];
    if (d_lo == 0 && g == 0) {
      a.part_ml[pi * 2 + 0] = m_run;
      a.part_ml[pi * 2 + 1] = l_tot;
    }
  }
}

// The scores half of the page for the prompt rows: S^T = K . Q^T per row
// (16 steps over 512 dims, two accumulation chains, K read in batches of 4
// fragments).
template <bool COMPRESSED, int NR>
__device__ __forceinline__ void global_rows_scores(f32x4 (&s)[NR][2], const uint8_t* pg, const bf16x8 (&qf)[NR][16],
                                                   int g, int l16) {
  using PG = GlobalPage<COMPRESSED>;
#pragma unroll
  for (int r = 0; r < NR; ++r) s[r][0] = s[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int hk = 0; hk < 4; ++hk) {
    bf16x8 kf[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      kf[k] = *reinterpret_cast<const bf16x8*>(pg + PG::k_off(4 * (4 * hk + k) + g, l16));
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
// blocks of 16 dims (V read in batches of 4 blocks).  V of tokens past p_v
// (slots past the workgroup's last row, possibly never written) is zeroed
// in the operand registers.
template <bool COMPRESSED, int NR>
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
#pragma unroll
    for (int b = 0; b < 4; ++b)
      vf[b] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vrow + 512 * (4 * bb + b))));
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

// Prompt rows (sequences with more than one query row: a new prompt's
// rows, or a chunk of one after a cached prefix, computed in the same step
// as the decode rows -- pegainfer "Gemma 4" page, Scheduling).  Row r of
// sequence s sits at position p_r = seq_len - q_len + r and attends keys
// 0 .. p_r.  kW = 8 / NR waves; wave (hb, rp) takes head block hb of rows
// NR rp .. NR rp + NR - 1 of the workgroup's kW NR / HB rows (NR = 1: two
// waves per SIMD; two rows per wave do not fit the registers), through a
// ring of NS pages that all waves fill.  No split: a row's whole range is
// one pass, and the output is written directly.  Items are (prompt
// sequence, row group), numbered compactly, a sequence's last groups
// (longest ranges) first.
template <bool COMPRESSED, int HB, int NR, int NS>
__global__ __launch_bounds__(64 * (8 / NR), 1) void global_prefill_kernel(GlobalAttnArgs a) {
  using PG = GlobalPage<COMPRESSED>;
  constexpr int kW = 8 / NR;                  // waves
  constexpr int kUnits = PG::kBytes / 1024;
  constexpr int kPerWave = kUnits / kW;       // units per wave per page ...
  constexpr int kPerWaveTail = kUnits % kW;   // ... the first kUnits % kW waves one more
  constexpr int kRows = kW * NR / HB;         // rows per workgroup
  static_assert(NR != 1 || kRows == global_prefill_rows(16 * HB), "the host's item count");
  static_assert(NS >= 2 && NS - 2 <= 4 && (kPerWave + 1) * (NS - 2) < 64, "ring depth");
  __shared__ __attribute__((aligned(16))) uint8_t ring[NS][PG::kBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = uniform_i32(tid >> 6);
  const int hb = HB == 2 ? (wv & 1) : 0;
  const int rp = HB == 2 ? (wv >> 1) : wv;
  const int g = lane >> 4, l16 = lane & 15;
  const int head = 16 * hb + l16;

  int s = -1, mg = 0, row0 = 0, q_len = 0, L = 0;
  {
    const int item = blockIdx.x;
    int base = 0;
    for (int c = 0; c < a.num_seqs; c += 64) {
      const int sl = c + lane;
      int cnt = 0, r0 = 0, ql = 0, len = 0;
      if (sl < a.num_seqs) {
        r0 = a.q_indptr[sl];
        ql = a.q_indptr[sl + 1] - r0;
        len = a.seq_lens[sl];
        if (ql > 1) cnt = (ql + kRows - 1) / kRows;
      }
      int incl = cnt;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int up = __shfl_up(incl, d, 64);
        incl += lane >= d ? up : 0;
      }
      const int total = __builtin_amdgcn_readlane(incl, 63);
      if (item < base + total) {
        const int ls = __builtin_ctzll(__ballot(base + incl > item));
        s = c + ls;
        const int nb = __builtin_amdgcn_readlane(cnt, ls);
        mg = nb - 1 - (item - (base + __builtin_amdgcn_readlane(incl, ls) - nb));
        row0 = __builtin_amdgcn_readlane(r0, ls);
        q_len = __builtin_amdgcn_readlane(ql, ls);
        L = __builtin_amdgcn_readlane(len, ls);
        break;
      }
      base += total;
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
  const int v_lane_off = global_v_lane_off<COMPRESSED>(0, g, l16);

  // software pipeline, one page deep: iteration i has pages i and i + 1 in
  // LDS; page i + 1's scores go out beside page i's weights and products
  if (nu > kPerWave) wait_groups_after<kPerWave + 1>(min(NS - 2, n - 1));
  else wait_groups_after<kPerWave>(min(NS - 2, n - 1));
  lds_barrier();
  f32x4 sc[NR][2];
  global_rows_scores<COMPRESSED, NR>(sc, ring[0], qf, g, l16);
  for (int i = 0; i < n; ++i) {
    if (nu > kPerWave) wait_groups_after<kPerWave + 1>(max(0, min(NS - 3, n - 2 - i)));
    else wait_groups_after<kPerWave>(max(0, min(NS - 3, n - 2 - i)));
    lds_barrier();   // pages i and i + 1 are in LDS for every wave; page i - 1 is done
    if (i + NS - 1 < n) issue_page(i + NS - 1);
    f32x4 sn[NR][2];
    global_rows_scores<COMPRESSED, NR>(sn, ring[min(i + 1, n - 1) % NS], qf, g, l16);
    global_rows_page<COMPRESSED, NR>(acc, m_run, l_run, ring[i % NS], sc, i * 16, pr, p_last, g, l16, v_lane_off,
                                     a.scale_log2);
#pragma unroll
    for (int r = 0; r < NR; ++r) { sc[r][0] = sn[r][0]; sc[r][1] = sn[r][1]; }
  }
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
}

// Cross-split reduce: M = max_i m_i, l = sum_i l_i 2^(m_i - M),
// out = sum_i acc_i 2^(m_i - M) / l, both sums in split order.  One
// workgroup per (sequence, q head), 128 threads: thread t owns output dims
// 4t .. 4t+3.  Every load of a chunk of 32 splits (each thread's acc
// quarter-rows, and (m, l) of split t by thread t) goes out at once, so a
// chunk costs one round trip; M and the weights are shared through LDS.
constexpr int kReduceChunk = 32;

__global__ __launch_bounds__(128) void global_split_reduce_kernel(ReduceArgs a) {
  __shared__ float sm_m[kReduceChunk], sm_l[kReduceChunk];
  const int s = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  int row = s;
  if (a.q_indptr) {
    row = a.q_indptr[s];
    if (a.q_indptr[s + 1] - row != 1) return;
  }
  const int nsplit = global_nsplit(cdiv_i(a.seq_lens[s], kPage));
  if (nsplit <= 1) return;
  const int64_t base = ((int64_t)s * a.num_q_heads + h) * a.max_splits;
  const float* pa = a.part_acc + base * kGD + 4 * t;
  const float* ml = a.part_ml + base * 2;
  float M = -INFINITY, lsum = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nsplit; c0 += kReduceChunk) {
    const int nc = min(kReduceChunk, nsplit - c0);
    f32x4 v[kReduceChunk];
#pragma unroll
    for (int i = 0; i < kReduceChunk; ++i)
      v[i] = i < nc ? *reinterpret_cast<const f32x4*>(pa + (int64_t)(c0 + i) * kGD) : f32x4{0.f, 0.f, 0.f, 0.f};
    if (t < nc) {
      const float2 x = *reinterpret_cast<const float2*>(ml + 2 * (c0 + t));
      sm_m[t] = x.x;
      sm_l[t] = x.y;
    }
    __syncthreads();
    // the running max over the splits so far; earlier chunks rescale once
    float mc = -INFINITY;
    for (int i = 0; i < nc; ++i) mc = fmaxf(mc, sm_m[i]);
    const float mnew = fmaxf(M, mc);
    if (mnew > M) {
      const float r = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - mnew);
      o *= r;
      lsum *= r;
      M = mnew;
    }
#pragma unroll
    for (int i = 0; i < kReduceChunk; ++i) {
      if (i < nc) {
        const float w = __builtin_amdgcn_exp2f(sm_m[i] - M);
        lsum += sm_l[i] * w;
        o += v[i] * w;
      }
    }
    __syncthreads();   // sm_m / sm_l are rewritten by the next chunk
  }
  *reinterpret_cast<f32x4*>(a.out + ((int64_t)row * a.num_q_heads + h) * kGD + 4 * t) = o / lsum;
}

}  // namespace

hipError_t launch_split_reduce(const ReduceArgs& a, int num_seqs, hipStream_t stream) {
  dim3 grid(num_seqs, a.num_q_heads), block(128);
  hipLaunchKernelGGL(global_split_reduce_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_global_decode(const GlobalAttnArgs& a, bool compressed, bool fp8, hipStream_t stream) {
  dim3 grid(a.max_splits * a.num_seqs), block(512);
  const bool h32 = a.num_q_heads == 32;
  constexpr int kNc = GW_GLOBAL_NP_C, kNf = GW_GLOBAL_NP_F, kNc8 = GW_GLOBAL_NP_C8, kNf8 = GW_GLOBAL_NP_F8;
  if (fp8) {
    if (compressed) {
      if (h32) hipLaunchKernelGGL((global_decode_kernel<true, 2, kNc8, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((global_decode_kernel<true, 1, kNc8, true>), grid, block, 0, stream, a);
    } else {
      if (h32) hipLaunchKernelGGL((global_decode_kernel<false, 2, kNf8, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((global_decode_kernel<false, 1, kNf8, true>), grid, block, 0, stream, a);
    }
  } else if (compressed) {
    if (h32) hipLaunchKernelGGL((global_decode_kernel<true, 2, kNc>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((global_decode_kernel<true, 1, kNc>), grid, block, 0, stream, a);
  } else {
    if (h32) hipLaunchKernelGGL((global_decode_kernel<false, 2, kNf>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((global_decode_kernel<false, 1, kNf>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_global_prefill(const GlobalAttnArgs& a, bool compressed, int max_q_len, hipStream_t stream) {
  // one workgroup per (prompt sequence, group of 8 / HB rows); the entry
  // point has checked that the count fits a grid
  const bool h32 = a.num_q_heads == 32;
  const long long items = prefill_items(a.num_rows, a.num_seqs, max_q_len, global_prefill_rows(a.num_q_heads));
  if (items == 0) return hipSuccess;
  if (items > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)items), block(512);
  if (compressed) {
    if (h32) hipLaunchKernelGGL((global_prefill_kernel<true, 2, 1, 4>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((global_prefill_kernel<true, 1, 1, 4>), grid, block, 0, stream, a);
  } else {
    if (h32) hipLaunchKernelGGL((global_prefill_kernel<false, 2, 1, 4>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((global_prefill_kernel<false, 1, 1, 4>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace gw
