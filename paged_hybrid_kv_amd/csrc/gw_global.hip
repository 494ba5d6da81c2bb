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
// contractions (heads x 16 tokens x 512 dims per page), so both run on MFMA
// with fp32 accumulation, in 16 x 16 blocks:
//   S^T (16 tokens x 16 heads) = K (16 x 512) . Q^T (512 x 16 heads)
//                                  -- v_mfma_f32_16x16x32_bf16, 16 steps
//   O^T (16 dims x 16 heads)  += V^T (16 x 16 tokens) . P^T (16 x 16 heads)
//                                  -- v_mfma_f32_16x16x16_bf16, per dim block
// The S^T result already sits in the lanes as the P^T operand wants it (lane
// l: head l % 16, tokens 4(l/16) .. +3), so the softmax of a page stays in
// the wave.
//
// Work split: one workgroup per (sequence, split) item, numbered compactly
// (workgroup b takes item b); a split is a balanced run of the row's pages
// (gw_plan.h).  A workgroup is two groups of four waves that take alternate
// pages of the split, each with its own online-softmax state, merged at the
// end.  Inside a group, wave w takes head block w % 2 (16 heads; with 16 q
// heads, the only block) and a slice of the output dims (256 dims per wave
// with 32 heads, 128 with 16); the waves of a head block split the score
// contraction's 512 dims the same way and add their partial scores through
// LDS, in a fixed order, so each score is computed once.  Pages stream
// straight from HBM into a ring of LDS page pairs (global_load_lds_dwordx4,
// each wave moving a quarter of its group's page), NP - 1 pairs in flight
// while one is read; after an LDS-only barrier each wave reads K (as stored)
// and V^T (through the gfx950 transposing LDS read ds_read_b64_tr_b16, or
// for an e4m3 page plain reads and a byte transpose across lanes) from its
// group's page.  On the
// row's last page, V of tokens past the row's position is zeroed in the
// operand registers and their scores are masked, so unwritten slots (possibly
// NaN) never reach the output.  P is rounded to bf16 for PV and the sum l
// adds exactly those rounded values.

#include "gw_device.h"
#include "gw_kernels.h"
#include "gw_plan.h"

namespace gw {
namespace {

constexpr int kGD = 512;

// LDS ring depth in page pairs, compressed / full record (3 x 40 KiB and
// 2 x 64 KiB: one workgroup per CU either way).
#ifndef GW_GLOBAL_NP_C
#define GW_GLOBAL_NP_C 3
#endif
#ifndef GW_GLOBAL_NP_F
#define GW_GLOBAL_NP_F 2
#endif
// e4m3 pages (10 and 16 KiB): 6 x 20 KiB and 3 x 32 KiB, q in a 32 KiB
// region of its own
#ifndef GW_GLOBAL_NP_C8
#define GW_GLOBAL_NP_C8 6
#endif
#ifndef GW_GLOBAL_NP_F8
#define GW_GLOBAL_NP_F8 3
#endif

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
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

// A page for one wave: its share of the scores of its 16 heads against the
// page's 16 tokens (global_page_scores), then, with the head block's partial
// scores added, the online-softmax update and the PV product into the wave's
// output-dim slice (global_page_update).  pg: the page in LDS; tok_page0:
// the position of the page's first token; p: the row's position (tokens past
// it are masked, and their V zeroed, so unwritten slots never reach the
// output).
// The wave's share of S^T = K . Q^T: the 4 HB 32-dim steps ks0 .. (the
// waves of a head block split the 512 dims between them; their partial
// sums are added through LDS).  The K fragments are read first (their LDS
// latencies overlap), then two accumulation chains; lane holds head l16,
// tokens 4g .. 4g+3.  e4m3 fragments (8 bytes) widen exactly to bf16 just
// before their product.
template <bool COMPRESSED, int HB, bool FP8 = false>
__device__ __forceinline__ f32x4 global_page_scores(const uint8_t* pg, const bf16x8 (&qf)[4 * HB], int ks0, int g,
                                                    int l16) {
  using PG = GlobalPage<COMPRESSED, FP8>;
  constexpr int kKs = 4 * HB;
  f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
  if constexpr (FP8) {
    uint2 kr[kKs];
#pragma unroll
    for (int k = 0; k < kKs; ++k) kr[k] = *reinterpret_cast<const uint2*>(pg + PG::k_off(4 * (ks0 + k) + g, l16));
    __builtin_amdgcn_sched_barrier(0);
    auto widen = [](uint2 r) __attribute__((always_inline)) {
      return __builtin_bit_cast(bf16x8, uint4{e4m3x2_to_bf16x2<false>(r.x), e4m3x2_to_bf16x2<true>(r.x),
                                              e4m3x2_to_bf16x2<false>(r.y), e4m3x2_to_bf16x2<true>(r.y)});
    };
#pragma unroll
    for (int k = 0; k < kKs; k += 2) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen(kr[k]), qf[k], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen(kr[k + 1]), qf[k + 1], s1, 0, 0, 0);
    }
  } else {
    bf16x8 kf[kKs];
#pragma unroll
    for (int k = 0; k < kKs; ++k) kf[k] = *reinterpret_cast<const bf16x8*>(pg + PG::k_off(4 * (ks0 + k) + g, l16));
    __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the products
#pragma unroll
    for (int k = 0; k < kKs; k += 2) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[k], qf[k], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[k + 1], qf[k + 1], s1, 0, 0, 0);
    }
  }
  return s0 + s1;
}

// The rest of a page for one wave, given the page's full scores sacc: the
// online-softmax update and the PV product into the wave's output-dim slice.
template <bool COMPRESSED, int HB, bool FP8 = false>
__device__ __forceinline__ void global_page_update(f32x4 (&acc)[8 * HB], float& m_run, float& l_run,
                                                   const uint8_t* pg, const f32x4 sacc, int tok_page0, int p, int g,
                                                   int l16, int v_lane_off, float scale_log2) {
  constexpr int kBlocks = 8 * HB;
  // ---- online softmax for head l16 over the page's 16 tokens
  const int tok0 = tok_page0 + 4 * g;
  float z[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) z[r] = (tok0 + r <= p) ? sacc[r] * scale_log2 : -INFINITY;
  const float mx = max_lanes_xor16_32(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
  const float mnew = fmaxf(m_run, mx);
  if (__any(mnew > m_run)) {
    const float alpha = mnew > m_run ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.f;
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) acc[b] *= alpha;
    l_run *= alpha;
  }
  m_run = mnew;
  const uint32_t p01 = pack_bf16(__builtin_amdgcn_exp2f(z[0] - m_run), __builtin_amdgcn_exp2f(z[1] - m_run));
  const uint32_t p23 = pack_bf16(__builtin_amdgcn_exp2f(z[2] - m_run), __builtin_amdgcn_exp2f(z[3] - m_run));
  l_run += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
  const s16x4 pb = __builtin_bit_cast(s16x4, uint2{p01, p23});

  // ---- O^T += V^T . P^T.  On the row's last page, V of tokens past p
  // (unwritten slots, possibly NaN) is zeroed in the operand registers.
  uint32_t vm0 = 0xffffffffu, vm1 = 0xffffffffu;
  if (tok_page0 + 15 > p) {
    vm0 = (tok0 + 0 <= p ? 0x0000ffffu : 0u) | (tok0 + 1 <= p ? 0xffff0000u : 0u);
    vm1 = (tok0 + 2 <= p ? 0x0000ffffu : 0u) | (tok0 + 3 <= p ? 0xffff0000u : 0u);
  }
  if constexpr (FP8) {
    // lane (g, 4a + c) reads dims 16b + 4a .. +3 of token 4g + c (4 bytes);
    // a byte transpose inside each quad of lanes (two DPP exchanges) leaves
    // lane c with dim 16b + 4a + c of tokens 4g .. 4g+3, which widen to bf16
    uint32_t vr[kBlocks];
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) vr[b] = *reinterpret_cast<const uint32_t*>(pg + v_lane_off + 256 * b);
    __builtin_amdgcn_sched_barrier(0);
    // byte selectors of v_perm_b32 (bytes 0-3: own word, 4-7: partner's):
    // step 1 with the xor-1 partner keeps bytes 0, 2 (even lane) or 1, 3
    // (odd lane) of both; step 2 with the xor-2 partner keeps the low
    // (lanes 0, 1) or high (lanes 2, 3) halves of both
    const int c = l16 & 3;
    const uint32_t sel1 = (c & 1) ? 0x03070105u : 0x06020400u;
    const uint32_t sel2 = (c & 2) ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) {
      const uint32_t x = vr[b];
      const uint32_t xp = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kQuadSwap1, 0xf, 0xf, false);
      const uint32_t y = __builtin_amdgcn_perm(xp, x, sel1);
      const uint32_t yp = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)y, kQuadSwap2, 0xf, 0xf, false);
      const uint32_t z = __builtin_amdgcn_perm(yp, y, sel2);
      const uint2 vv = uint2{e4m3x2_to_bf16x2<false>(z) & vm0, e4m3x2_to_bf16x2<true>(z) & vm1};
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vv), pb, acc[b], 0, 0, 0);
    }
  } else {
    lds_u8* vrow = (lds_u8*)pg + v_lane_off;
    uint2 vf[kBlocks];
#pragma unroll
    for (int b = 0; b < kBlocks; ++b)
      vf[b] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vrow + 512 * b)));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) {
      uint2 vv = vf[b];
      vv.x &= vm0;
      vv.y &= vm1;
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vv), pb, acc[b], 0, 0, 0);
    }
  }
}

// Byte offset, inside a page, of what lane (g, l16) names in the transposing
// read of V for dims d_lo .. (lane (g, e, q) names token 4g + e, dims
// d_lo + 4q .. +3, and receives dim d_lo + l16 of tokens 4g .. 4g+3).
// e4m3 (FP8): lane (g, 4a + c) reads dims d_lo + 4a .. +3 of token 4g + c.
template <bool COMPRESSED, bool FP8 = false>
__device__ __forceinline__ int global_v_lane_off(int d_lo, int g, int l16) {
  if constexpr (FP8)
    return GlobalPage<COMPRESSED, FP8>::kVOff + ((d_lo >> 4) * 16 + 4 * g + (l16 & 3)) * 16 + 4 * (l16 >> 2);
  const int t_rd = 4 * g + (l16 >> 2);
  const int dd = d_lo + 4 * (l16 & 3);
  return GlobalPage<COMPRESSED>::kVOff + ((dd >> 3) * 16 + t_rd) * 16 + (dd & 7) * 2;
}

// One workgroup = two groups of four waves.  Group q (0, 1) takes the pages
// 2j + q of the split: in every step j the two groups work on the two pages
// of pair j side by side (one wave of each group per SIMD, so the phases of
// one overlap the other's), each with its own online-softmax state; the two
// states merge once at the end, group 1 into group 0, in that order.
// NP: page pairs in the LDS ring (NP - 1 pairs in flight while one is read).
// FP8: e4m3 pages, widened to bf16 as they are read from LDS; q then has an
// LDS region of its own after the ring, and a 10 KiB compressed page moves
// as 3 + 3 + 2 + 2 units (waves 0, 1 take one unit of the last two each).
template <bool COMPRESSED, int HB, int NP, bool FP8 = false>
__global__ __launch_bounds__(512, 1) void global_decode_kernel(GlobalAttnArgs a) {
  using PG = GlobalPage<COMPRESSED, FP8>;
  constexpr int kUnits = PG::kBytes / 1024;   // 1 KiB transfer units per page
  constexpr int kPerWave = (kUnits + 3) / 4;  // most units a wave moves per page
  constexpr int kExtra = kUnits - 4 * (kUnits / 4);   // waves below kExtra move one more
  constexpr int kBlocks = 8 * HB;             // 16-dim output blocks per wave
  constexpr int kRingBytes = NP * 2 * PG::kBytes;
  static_assert(NP >= 2 && kPerWave * (NP - 2) < 64 && NP - 2 <= 4, "ring depth");
  static_assert(kRingBytes >= 4 * kBlocks * 64 * 16 + 4 * 64 * 8, "the ring holds the group merge");
  static_assert(FP8 || 2 * PG::kBytes >= 32 * 1024, "a ring slot holds q");
  constexpr int kXsOff = kRingBytes + (FP8 ? 32 * 1024 : 0);   // partial scores, [wave][lane] f32x4
  __shared__ __attribute__((aligned(16))) uint8_t smem[kXsOff + 8 * 64 * 16];
  uint8_t(*ring)[2][PG::kBytes] = reinterpret_cast<uint8_t(*)[2][PG::kBytes]>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = uniform_i32(tid >> 6);
  const int grp = wv >> 2, w = wv & 3;
  const int hb = HB == 2 ? (w & 1) : 0;
  const int d_lo = HB == 2 ? 256 * (w >> 1) : 128 * w;
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
  if (append_here && wv == 0)
    rec = global_record_lane(a.v_new + (int64_t)row * kGD, a.v_new + (int64_t)row * kGD, a.rope_cos, a.rope_sin, p, lane);
  asm volatile("" ::"v"(ptv0), "v"(ptv1), "v"(ptv2), "v"(ptv3));
  if (append_here && wv == 0)
    put_global_record_as<COMPRESSED, FP8>(const_cast<uint8_t*>(a.pool) + (int64_t)phys(n - 1) * a.page_bytes, rec,
                                          p & 15, lane);

  // ---- q into LDS by direct transfers, ahead of the pages, in ring slot
  // NP - 1 (free until the loop's first transfer): 1 KiB per head, the
  // row's 16-byte chunk c of head h stored at chunk c ^ (h % 8), so that the
  // Q^T operand reads below hit distinct banks.  Wave wv moves heads
  // 2 HB wv .. +2 HB - 1; lane i fetches the chunk that lands at position i.
  uint8_t* qs = FP8 ? smem + kRingBytes : &ring[NP - 1][0][0];
  {
    const uint32_t qs_lds = uniform_i32((int)lds_address(qs));
#pragma unroll
    for (int i = 0; i < 2 * HB; ++i) {
      const int h = 2 * HB * wv + i;
      dma16_to_lds(a.q + ((int64_t)row * a.num_q_heads + h) * kGD + 8 * (lane ^ (h & 7)),
                   qs_lds + (uint32_t)(h * 1024));
    }
  }

  // ---- transfers: group q moves page 2j + q of pair j, wave w of the group
  // the units [kPerWave w, kPerWave (w + 1)) of the page (1 KiB each), so
  // the LDS copy has the pool's layout.  An odd split's last pair repeats
  // its last page as the second one; that copy is never computed on.  The
  // loop's waits count transfers only; the appending wave's pool stores and
  // the q transfers are older than all of them, so they are covered too.
  // wave w moves units kUnits/4 * w + u, and, below kExtra, unit 4 (kUnits/4) + w
  constexpr int kEven = kUnits / 4;
  const int my_units = kEven + (w < kExtra ? 1 : 0);
  const uint32_t ring_base = uniform_i32((int)lds_address(&ring[0][0][0])) + (uint32_t)(grp * PG::kBytes);
  auto issue_pair = [&](int j) __attribute__((always_inline)) {
    const int i = min(2 * j + grp, n - 1);
    const uint8_t* src = a.pool + (int64_t)phys(i) * a.page_bytes + 16 * lane;
    const uint32_t dst = ring_base + (uint32_t)((j % NP) * 2 * PG::kBytes);
#pragma unroll
    for (int u = 0; u < kEven; ++u) dma16_to_lds(src + 1024 * (kEven * w + u), dst + 1024 * (kEven * w + u));
    if (kExtra > 0 && w < kExtra) dma16_to_lds(src + 1024 * (4 * kEven + w), dst + 1024 * (4 * kEven + w));
  };
  // at most k pairs' transfers of this wave left in flight
  auto wait_pairs_after = [&](int k) __attribute__((always_inline)) {
    if (kExtra > 0 && my_units == kEven) wait_groups_after<(kExtra > 0 ? kEven : kPerWave)>(k);
    else wait_groups_after<kPerWave>(k);
  };
#pragma unroll
  for (int j = 0; j < NP - 1; ++j)
    if (j < n_pairs) issue_pair(j);

  // Q^T operand for the wave's part of the score dims (part `part` of the
  // 4 / HB waves of its head block): head 16hb + l16, dims 32ks + 8g .. +7
  // (16-byte chunk 4ks + g), once every wave's q transfers (older than its
  // page transfers) are in
  constexpr int kKs = 4 * HB;
  const int part = HB == 2 ? (w >> 1) : w;
  wait_pairs_after(min(NP - 1, n_pairs));
  lds_barrier();
  bf16x8 qf[kKs];
#pragma unroll
  for (int k = 0; k < kKs; ++k) {
    const int ks = part * kKs + k;
    qf[k] = *reinterpret_cast<const bf16x8*>(qs + head * 1024 + (((4 * ks + g) ^ (head & 7)) * 16));
  }
  f32x4* xs = reinterpret_cast<f32x4*>(smem + kXsOff);

  f32x4 acc[kBlocks];
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int v_lane_off = global_v_lane_off<COMPRESSED, FP8>(d_lo, g, l16);

  for (int j = 0; j < n_pairs; ++j) {
    wait_pairs_after(min(NP - 2, n_pairs - 1 - j));
    lds_barrier();   // pair j is in LDS for every wave; pair j - 1 is done
    if (j + NP - 1 < n_pairs) issue_pair(j + NP - 1);
    if (append_here && j == ((n - 1) >> 1)) {
      if (wv == 0) put_global_record_as<COMPRESSED, FP8>(&ring[j % NP][(n - 1) & 1][0], rec, p & 15, lane);
      lds_barrier();
    }
    // both groups pass the exchange barrier, also a group with no page in
    // the split's last pair
    const int i = 2 * j + grp;
    const bool live = i < n;
    const uint8_t* pg = ring[j % NP][grp];
    if (live) xs[wv * 64 + lane] = global_page_scores<COMPRESSED, HB, FP8>(pg, qf, part * kKs, g, l16);
    lds_barrier();
    if (live) {
      // the head block's partial scores, added in part order by every wave
      const f32x4* xh = xs + (4 * grp + hb) * 64 + lane;
      f32x4 sacc;
      if constexpr (HB == 2) sacc = xh[0] + xh[2 * 64];
      else sacc = (xh[0] + xh[64]) + (xh[2 * 64] + xh[3 * 64]);
      global_page_update<COMPRESSED, HB, FP8>(acc, m_run, l_run, pg, sacc, (pg0 + i) * 16, p, g, l16, v_lane_off,
                                              a.scale_log2);
    }
  }

  // ---- merge group 1 into group 0 through LDS (the ring is free now):
  // M = max(m0, m1), acc = acc0 2^(m0 - M) + acc1 2^(m1 - M), same for l
  lds_barrier();
  float* xa = reinterpret_cast<float*>(&ring[0][0][0]) + (w * kBlocks * 64 + lane) * 4;
  float* xm = reinterpret_cast<float*>(&ring[0][0][0]) + 4 * kBlocks * 64 * 4 + (w * 64 + lane) * 2;
  if (grp == 1) {
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) *reinterpret_cast<f32x4*>(xa + b * 256) = acc[b];
    xm[0] = m_run;
    xm[1] = l_run;
  }
  lds_barrier();
  if (grp == 1) return;
  {
    const float m1 = xm[0], l1 = xm[1];
    const float M = fmaxf(m_run, m1);
    const float s0 = __builtin_amdgcn_exp2f(m_run - M);
    const float s1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) acc[b] = acc[b] * s0 + *reinterpret_cast<const f32x4*>(xa + b * 256) * s1;
    l_run = l_run * s0 + l1 * s1;
    m_run = M;
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
