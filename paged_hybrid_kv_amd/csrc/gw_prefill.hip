// Local-family attention of prompt rows (sequences with more than one query
// row in the call): sliding window, head dim 256, grouped query heads, bf16
// or e4m3 pool.
//
// What is computed (pegainfer "Gemma 4" page, Scheduling: prompt rows share
// the step with the decode rows; intro and
// Architecture notes for the window and the grouped heads): row r of
// sequence s sits at position p_r = seq_len - q_len + r; each q head h of
// KV head g = h / G attends the keys j in [max(0, p_r - W + 1), p_r].
//
// With many rows per KV head the score and value steps are dense
// contractions, so both run on MFMA over "query vectors" (a row and one head
// of its group), 16 to a block: lane column l16 of block qb of wave w is
// query vector v = 16 QB w + 16 qb + l16 (row r_first + v / G, head v % G).
// The keys go by in steps of 32 tokens (two pages):
//   S^T (16 tokens x 16 q vectors) = K (16 x 256) . Q^T (256 x 16)
//         -- v_mfma_f32_16x16x32_bf16, 8 steps, per page and query block
//   O^T (16 dims x 16 q vectors)  += V^T (16 x 32 tokens) . P^T (32 x 16)
//         -- v_mfma_f32_16x16x32_bf16, per 16-dim block and query block
// where lane (l16, gq) holds the scores of tokens 4 gq .. +3 of each page,
// which it also supplies as the PV step's k slots 8 gq .. +7, so P never
// leaves the lane.  A workgroup of 8 / QB waves (QB query blocks each; 128
// query vectors in all) takes 128 / G consecutive rows of one (sequence,
// KV head) and streams the pages of their union range,
// [max(0, p_first - W + 1), p_last], through an LDS ring (direct
// global->LDS transfers, every wave moving its share of every page), so K/V
// are read once per 128 query vectors.  With one block per wave there are
// two waves per SIMD, so one wave's weights (VALU) and reads (LDS) overlap
// the other's products; that beats the halved LDS traffic of two blocks per
// wave at one wave per SIMD.  Each lane masks its own query vectors'
// windows; V of tokens outside the union range (slots that may never have
// been written) is zeroed in LDS on the range's edge steps.  e4m3 codes
// convert to bf16 exactly (v_cvt_scalef32_pk_bf16_fp8, scale 1), so the
// products are the same as on the bf16 values.  P is rounded to bf16 for
// PV and the sum l adds exactly those rounded values.  A prompt that lies
// inside one window has row blocks whose ranges grow with the block; its
// workgroups fold (half of an early block with the same half of the
// mirrored late block), so they stream about the same work, and waves
// skip the steps past their own rows.  Workgroups are
// numbered compactly over the prompt sequences' row blocks, level by level
// (every sequence's last block first, then every sequence's second last,
// ...: the longest ranges of the call first), with the KV head as the
// fastest index (so one head's blocks share an XCD when there are eight
// heads).

#include "gw_device.h"
#include "gw_kernels.h"
#include "gw_plan.h"

namespace gw {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
// A read-only int32 array read through the constant address space, so that
// uniform reads become scalar loads.
typedef const __attribute__((address_space(4))) int32_t* CI32P;

// One (page, KV head) record as the prefill kernel keeps it in LDS.  The
// transfers move 16-byte chunks, 1 KiB units at a time, and place them so
// that a fragment read of 16 lanes (bf16 K) or of the whole wave (bf16 V)
// touches every LDS bank once: K unit chunk (t, c) (token t, quarter c)
// sits at position 4 t + (c ^ (t / 4)), and chunk c of V unit u at
// c ^ (4 ((u / 2) % 4)).  e4m3 records keep the pool's layout.
template <bool FP8>
struct LocalHead {
  static constexpr int kBytes = FP8 ? 8192 : 16384;   // K block + V block of one KV head
  static constexpr int kVOff = kBytes / 2;
  static constexpr int kKUnits = kVOff / 1024;
  // byte offset, inside unit U of the record, of the chunk that the
  // transfer lane `lane` places at its own position
  __device__ static __forceinline__ int src_chunk_off(int U, int lane) {
    if constexpr (FP8) {
      return 16 * lane;
    } else {
      if (U < kKUnits) {
        const int t = lane >> 2;
        return 16 * (4 * t + ((lane & 3) ^ (t >> 2)));
      }
      return 16 * (lane ^ (4 * (((U - kKUnits) >> 1) & 3)));
    }
  }
  // K operand: token t, dims 32 ks + 8 gq .. +7, as 8 bf16
  __device__ static __forceinline__ bf16x8 k_frag(const uint8_t* pg, int ks, int gq, int t) {
    if constexpr (!FP8) {
      const int k = 4 * (ks & 1) + gq, c = ks >> 1;
      return *reinterpret_cast<const bf16x8*>(pg + k * 1024 + (4 * t + (c ^ (t >> 2))) * 16);
    } else {
      const int k = 2 * (ks & 1) + (gq >> 1), c = ks >> 1;
      const uint2 w = *reinterpret_cast<const uint2*>(pg + ((k * 16 + t) * 4 + c) * 16 + 8 * (gq & 1));
      return __builtin_bit_cast(bf16x8, uint4{e4m3x2_to_bf16x2<false>(w.x), e4m3x2_to_bf16x2<true>(w.x),
                                              e4m3x2_to_bf16x2<false>(w.y), e4m3x2_to_bf16x2<true>(w.y)});
    }
  }
  // Zero, in the LDS copies of a step's two pages, V of every slot whose
  // token (tok0 + slot, page 1 from tok0 + 16) lies outside [lo, hi];
  // thread tid of 256 takes one dim (bf16) or one dword of codes (e4m3).
  __device__ static __forceinline__ void zero_v_outside(uint8_t* pg0, uint8_t* pg1, int tok0, int lo, int hi,
                                                        int tid) {
    for (int t = 0; t < 32; ++t) {
      const int pos = tok0 + t;
      if (pos >= lo && pos <= hi) continue;
      uint8_t* vb = (t < 16 ? pg0 : pg1) + kVOff;
      const int slot = t & 15;
      if constexpr (!FP8) {
        const int u = slot >> 1;
        const int d = tid;   // dim
        reinterpret_cast<uint16_t*>(vb + u * 1024 + (d ^ (16 * ((u >> 1) & 3))) * 4)[slot & 1] = 0;
      } else {
        const int u = slot >> 2;   // quad of slots, dword per dim
        const int d = tid;
        vb[u * 1024 + d * 4 + (slot & 3)] = 0;
      }
    }
  }
  // V^T operand: dim d, tokens 4 gq .. 4 gq + 3, as 4 bf16 (two dwords)
  __device__ static __forceinline__ uint2 v_frag(const uint8_t* pg, int d, int gq) {
    if constexpr (!FP8) {
      const uint8_t* b = pg + kVOff + (2 * gq) * 1024 + (d ^ (16 * gq)) * 4;
      return uint2{*reinterpret_cast<const uint32_t*>(b), *reinterpret_cast<const uint32_t*>(b + 1024)};
    } else {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(pg + kVOff + ((gq * 64 + (d >> 2)) * 4 + (d & 3)) * 4);
      return uint2{e4m3x2_to_bf16x2<false>(w), e4m3x2_to_bf16x2<true>(w)};
    }
  }
};

// Largest excess, in base-2 exponent, of a score over the running reference
// max before the reference moves (so unnormalised weights stay <= 2^8).
constexpr float kLazyMax = 8.f;

// Query blocks (16 query vectors) per wave: 8 / kPrefillQB waves per workgroup.
#ifndef GW_PREFILL_QB
#define GW_PREFILL_QB 1
#endif
constexpr int kPrefillQB = GW_PREFILL_QB;


template <int G, bool FP8, int NS, int QB>
__global__ __launch_bounds__(64 * (8 / QB), 1) void local_prefill_kernel(LocalAttnArgs a) {
  using LH = LocalHead<FP8>;
  constexpr int kUnits = LH::kBytes / 1024;    // 1 KiB transfer units per (page, head)
  constexpr int kWaves = 8 / QB;               // waves per workgroup, QB query blocks each
  constexpr int kPerWavePage = kUnits / kWaves;   // units a wave moves of each page
  constexpr int kPerStep = 2 * kPerWavePage;   // transfers per wave per two-page step
  constexpr int kRows = local_prefill_rows(G);
  static_assert(NS >= 3 && NS - 2 <= 4 && kPerStep * (NS - 2) < 64, "ring depth");
  __shared__ __attribute__((aligned(16))) uint8_t ring[NS][2][LH::kBytes];

  // workgroup b: KV head b % Hkv of item b / Hkv (the head fastest)
  const int gk = (int)blockIdx.x % a.num_kv_heads;
  const int tid = threadIdx.x, lane = tid & 63;
  // trace slots (row kTracePrefillRow + b): 0 XCD | row block << 8 | KV
  // head << 16 | sequence << 32, 1 steps, 2 entry, 3 first step in LDS,
  // 4 wave 0's loop done, 5 iteration 1 open, 6 last iteration open, 7 exit,
  // 8 + w wave w's loop done
  const int trow = kTracePrefillRow + (int)blockIdx.x;
  GW_TRACE_AT(a, trow, 2, tid == 0);
  const int w = uniform_i32(tid >> 6);
  const int gq = lane >> 4, l16 = lane & 15;

  // ---- work item: the call's (prompt sequence, row block) items, level by
  // level (every sequence's last block -- the longest range -- first)
  int s = -1, rb = 0, row0 = 0, q_len = 0, L = 0;
  {
    PromptItem it;
    if (prompt_item(a.q_indptr, a.seq_lens, a.num_seqs, kRows, (int)blockIdx.x / a.num_kv_heads, lane, it)) {
      s = it.s;
      rb = it.grp;
      row0 = it.row0;
      q_len = it.q_len;
      L = it.len;
    }
  }
  if (s < 0) return;
  s = uniform_i32(s);
  rb = uniform_i32(rb);
  row0 = uniform_i32(row0);
  q_len = uniform_i32(q_len);
  L = uniform_i32(L);

  // The item's rows: two halves of kRows / 2 rows, the first taken by
  // waves 0 .. kWaves / 2 - 1, the second by the others.  Normally the two
  // halves of row block rb.  A prompt that lies inside one window (every
  // row attends from key 0: the ranges grow with the row block) folds:
  // item rb < 2 (nb / 2) takes half rb % 2 of block rb / 2 and the same
  // half of block nb - 1 - rb / 2, and the middle block of an odd count
  // stays whole, so the prompt's items stream about the same work; a wave
  // skips the steps past its own rows.
  const int pos0 = L - q_len;
  constexpr int kHalf = kRows / 2;
  constexpr int kHalfWaves = kWaves / 2;
  const int nb = cdiv_i(q_len, kRows);
  const bool in_window = L <= a.window;
  const bool fold = in_window && rb < 2 * (nb / 2);   // uniform
  const int blk = in_window ? nb / 2 : rb;             // the whole block of an item that does not fold
  const int ra = fold ? (rb >> 1) * kRows + (rb & 1) * kHalf : blk * kRows;
  const int rbh = fold ? (nb - 1 - (rb >> 1)) * kRows + (rb & 1) * kHalf : blk * kRows + kHalf;
  // rows r_first .. r_last (the first half's first row, the last valid
  // row of either half) at positions pos0 + r; their union range
  // [lo_first, p_last] covers pages pg_lo .. pg_lo + n_pages - 1, walked in
  // steps of two pages (an odd count's last step repeats its last page as
  // the second, every token of which lies past p_last)
  const int r_first = ra;
  const int r_last = rbh < q_len ? min(rbh + kHalf, q_len) - 1 : min(ra + kHalf, q_len) - 1;
  const int p_last = pos0 + r_last;
  const int lo_first = max(0, pos0 + r_first - a.window + 1);
  const int pg_lo = lo_first >> 4;
  const int n_pages = (p_last >> 4) - pg_lo + 1;
  const int n_steps = (n_pages + 1) >> 1;
  // this wave's rows: w_first .. w_last (valid rows only; none when
  // w_last < w_first), which attend [lo_max, p_min] at least, and its last
  // step
  const int wh = w % kHalfWaves;
  const int wbase = w < kHalfWaves ? ra : rbh;
  const int w_first = wbase + (16 * QB * wh) / G;
  const int w_last = min(min(wbase + (16 * QB * wh + 16 * QB - 1) / G, wbase + kHalf - 1), q_len - 1);
  const int lo_max = max(0, pos0 + w_last - a.window + 1);
  const int p_min = pos0 + w_first;
  const int last_step = w_last < w_first ? -1 : (((pos0 + w_last) >> 4) - pg_lo) >> 1;
  GW_TRACE_VAT(a, trow, 0, tid == 0, GW_TRACE_XCC() | (uint64_t)rb << 8 | (uint64_t)gk << 16 | (uint64_t)s << 32);
  GW_TRACE_VAT(a, trow, 1, tid == 0, n_steps);

  // this lane's query vectors, v = 16 QB (w % (kWaves / 2)) + 16 qb + l16
  // of its half: row (first row of the half) + v / G, head v % G of the
  // group; each masks its own window (a row past the prompt computes on
  // r_last's query and position and is not written)
  int pq[QB], loq[QB], rq[QB];
  bool rok[QB];
  bf16x8 qf[QB][8];   // Q^T operand: dims 32 ks + 8 gq .. +7
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int v = 16 * QB * wh + 16 * qb + l16;
    const int r = wbase + v / G;
    rok[qb] = r < q_len;
    const int rr = rok[qb] ? r : r_last;
    rq[qb] = r;
    pq[qb] = pos0 + rr;
    loq[qb] = max(0, pq[qb] - a.window + 1);
    const uint16_t* qp = a.q + ((int64_t)(row0 + rr) * a.num_q_heads + gk * G + v % G) * 256 + 8 * gq;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[qb][ks] = __builtin_bit_cast(bf16x8, ld16_cached(qp + 32 * ks));
  }
  // page ids come through the scalar cache (the page table is read-only
  // during the call), one uniform load per page as its transfer is issued
  const CI32P pt = (CI32P)(a.page_table + (int64_t)s * a.pt_stride + pg_lo);
  // q is not waited for before the transfers: the compiler's own wait at the
  // first product (it does not see the transfers) holds for those already
  // issued too, which the first step needs anyway

  const uint32_t ring_base = uniform_i32((int)lds_address(&ring[0][0][0])) + (uint32_t)(1024 * kPerWavePage * w);
  const int64_t head_off = (int64_t)gk * a.head_bytes + 1024 * kPerWavePage * w;
  int src_off[kPerWavePage];
#pragma unroll
  for (int u = 0; u < kPerWavePage; ++u) src_off[u] = 1024 * u + LH::src_chunk_off(kPerWavePage * w + u, lane);
  auto issue_step = [&](int j) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint8_t* src = a.pool + (int64_t)pt[min(2 * j + h, n_pages - 1)] * a.page_bytes + head_off;
      const uint32_t dst = ring_base + (uint32_t)(((j % NS) * 2 + h) * LH::kBytes);
#pragma unroll
      for (int u = 0; u < kPerWavePage; ++u) dma16_to_lds(src + src_off[u], dst + 1024 * u);
    }
  };
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < n_steps) issue_step(j);

  f32x4 acc[QB][16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int b = 0; b < 16; ++b) acc[qb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[QB];
  f32x4 lacc[QB];   // l, in every element
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    lacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8 kOnes = __builtin_bit_cast(bf16x8, uint4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});

  // ---- S^T = K . Q^T for both pages (tb) and both query blocks (qb) of a
  // step in the ring: all 16 K fragments first, then four interleaved
  // accumulation chains
  auto scores = [&](int j, f32x4 (&sc)[2][QB]) __attribute__((always_inline)) {
    const uint8_t* pg0 = ring[j % NS][0];
    const uint8_t* pg1 = ring[j % NS][1];
    bf16x8 kf[2][8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kf[0][ks] = LH::k_frag(pg0, ks, gq, l16);
      kf[1][ks] = LH::k_frag(pg1, ks, gq, l16);
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[tb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sc[tb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[tb][ks], qf[qb][ks], sc[tb][qb], 0, 0, 0);
  };

  // Software pipeline, one step deep: iteration j turns step j's scores
  // (computed in iteration j - 1) into weights on VALU while step j + 1's
  // scores run on MFMA, then adds step j's PV.  Steps j and j + 1 are in
  // LDS during iteration j, so NS - 2 steps are in flight; step j - 1's
  // slot is refilled once every wave is past iteration j - 1.
  wait_groups_after<kPerStep>(min(n_steps - 1, NS - 2));
  lds_barrier();
  GW_TRACE_AT(a, trow, 3, tid == 0);
  f32x4 sc[2][QB];
  if (last_step >= 0) scores(0, sc);
  for (int j = 0; j < n_steps; ++j) {
    const int jn = min(j + 1, n_steps - 1);   // the last iteration recomputes its own step's scores, unused
    wait_groups_after<kPerStep>(max(0, min(n_steps - 2 - j, NS - 3)));
    lds_barrier();   // step j + 1 is in LDS for every wave; step j - 1 is done
    GW_TRACE_AT(a, trow, 5, tid == 0 && j == 1);
    GW_TRACE_AT(a, trow, 6, tid == 0 && j == n_steps - 1);
    if (j + NS - 1 < n_steps) issue_step(j + NS - 1);
    const uint8_t* pg0 = ring[j % NS][0];
    const uint8_t* pg1 = ring[j % NS][1];
    const int tok0 = (pg_lo + 2 * j) * 16;
    // At the union range's edges, V of the step's tokens outside it (slots
    // that may never have been written) is zeroed in LDS before any wave
    // reads it (its K was read a step earlier; those scores are masked).
    if (tok0 < lo_first || tok0 + 31 > p_last) {
      if (tid < 256) LH::zero_v_outside(ring[j % NS][0], ring[j % NS][1], tok0, lo_first, p_last, tid);
      lds_barrier();
    }
    // a wave whose rows end before this step only keeps the ring moving
    if (j > last_step) continue;

    // ---- scaled scores z; a step inside every row's window of the wave
    // (the common case) takes no masks (rows past the prompt compute on
    // r_last's q and are not written)
    const bool full = tok0 >= lo_max && tok0 + 31 <= p_min;
    float z[QB][8];
    if (full) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < 8; ++i) z[qb][i] = sc[i >> 2][qb][i & 3] * a.scale_log2;
    } else {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        // this query vector's keys, relative to the step: [lo, hi] (empty past r_last)
        const int lo = rok[qb] ? loq[qb] - tok0 : 64;
        const int hi = pq[qb] - tok0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int t = 16 * (i >> 2) + 4 * gq + (i & 3);
          z[qb][i] = ((t >= lo) & (t <= hi)) ? sc[i >> 2][qb][i & 3] * a.scale_log2 : -INFINITY;
        }
      }
    }
    // The reference max moves only when a score passes it by more than
    // kLazyMax (weights then stay below 2^kLazyMax), so the accumulators --
    // in AGPRs -- are rescaled rarely after the first step; whether any
    // lane needs it is known from its own eight scores, and only then are
    // the row maxima formed across the four lanes of each query vector.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = fmaxf(fmaxf(fmaxf(z[qb][0], z[qb][1]), fmaxf(z[qb][2], z[qb][3])),
                       fmaxf(fmaxf(z[qb][4], z[qb][5]), fmaxf(z[qb][6], z[qb][7])));
      if (__any(mx > m_run[qb] + kLazyMax)) {
        mx = max_lanes_xor16_32(mx);
        const bool up = mx > m_run[qb] + kLazyMax;
        const float alpha = up ? __builtin_amdgcn_exp2f(m_run[qb] - mx) : 1.f;
#pragma unroll
        for (int b = 0; b < 16; ++b) acc[qb][b] *= alpha;
        lacc[qb] *= alpha;
        m_run[qb] = up ? mx : m_run[qb];
      }
    }

    // ---- from here on one block without branches, so that the next
    // step's score MFMAs interleave with this step's weights (VALU) and V
    // reads (LDS).  A query vector with no key yet has m = -inf and only
    // -inf scores: its reference is taken as 0 so that its weights are 0.
    f32x4 sn[2][QB];
    scores(jn, sn);
    bf16x8 pb[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mref = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
      uint32_t pw[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        pw[k] = pack_bf16(__builtin_amdgcn_exp2f(z[qb][2 * k] - mref), __builtin_amdgcn_exp2f(z[qb][2 * k + 1] - mref));
      pb[qb] = __builtin_bit_cast(bf16x8, uint4{pw[0], pw[1], pw[2], pw[3]});
      // l += the rounded weights, summed over the 32 tokens by MFMA (ones . P^T)
      lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kOnes, pb[qb], lacc[qb], 0, 0, 0);
    }
    uint4 vf[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const uint2 v0 = LH::v_frag(pg0, 16 * b + l16, gq), v1 = LH::v_frag(pg1, 16 * b + l16, gq);
      vf[b] = uint4{v0.x, v0.y, v1.x, v1.y};
    }

    // ---- O^T += V^T . P^T over the 32 tokens: lane (l16, gq) gives dim
    // 16 b + l16 of the same eight tokens
#pragma unroll
    for (int b = 0; b < 16; ++b)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        acc[qb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf[b]), pb[qb], acc[qb][b], 0, 0, 0);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[tb][qb] = sn[tb][qb];
  }

  GW_TRACE_AT(a, trow, 4, tid == 0);
  GW_TRACE_AT(a, trow, 8 + w, lane == 0);

  // ---- write: lane holds query vector l16 of each block, dims 16 b + 4 gq .. +3
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = lacc[qb][0];
    if (!rok[qb]) continue;
    const int v = 16 * QB * wh + 16 * qb + l16;
    float* op = a.out + ((int64_t)(row0 + rq[qb]) * a.num_q_heads + gk * G + v % G) * 256 + 4 * gq;
    const float inv = 1.f / l_tot;
    // streaming stores: nothing in this step reads the rows' outputs again,
    // so they go out to memory now, while this kernel leaves HBM idle,
    // instead of sitting dirty in the caches until the next decode kernel's
    // stream evicts them
#pragma unroll
    for (int b = 0; b < 16; ++b) __builtin_nontemporal_store(acc[qb][b] * inv, reinterpret_cast<f32x4*>(op + 16 * b));
  }
  GW_TRACE_AT(a, trow, 7, tid == 0);
}

}  // namespace

hipError_t launch_local_prefill(const LocalAttnArgs& a, int group, bool fp8, int max_q_len,
                                hipStream_t stream) {
  // one workgroup per (item, KV head); the entry point has checked that the
  // count fits a grid
  const long long n = prefill_items(a.num_rows, a.num_seqs, max_q_len, local_prefill_rows(group)) * a.num_kv_heads;
  if (n == 0) return hipSuccess;
  if (n > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)n), block(64 * (8 / kPrefillQB));
#define GW_PREFILL_CASE(G_, F_)                                                                     \
  if (group == G_ && fp8 == F_) {                                                                   \
    hipLaunchKernelGGL((local_prefill_kernel<G_, F_, 3, kPrefillQB>), grid, block, 0, stream, a);   \
    return hipGetLastError();                                                                       \
  }
  GW_PREFILL_CASE(1, false) GW_PREFILL_CASE(2, false) GW_PREFILL_CASE(4, false)
  GW_PREFILL_CASE(1, true) GW_PREFILL_CASE(2, true) GW_PREFILL_CASE(4, true)
#undef GW_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace gw
