// Local-family paged decode attention (sliding window, head dim 256, grouped
// query heads), with the decode rows' own K/V append and the cross-split
// reduce fused in.
//
// What is computed (pegainfer "Gemma 4" page, intro and Architecture notes;
// pegainfer PR #1012, Description, for the e4m3 pool): for each decode row of
// sequence s at position p = seq_len - 1 and each q head h of KV head
// g = h / G, softmax over the keys j in [max(0, p - W + 1), p] of
// scale * q_h . K_j, applied to V_j, with K/V read from 16-token pages.
// When the call carries the rows' new K/V, the token at p is rotated and
// stored first (the prep step), exactly as gw_kv_append stores it.
//
// Work split: one workgroup per (split, KV head, sequence), numbered
// split-major; a split is a balanced run of the row's range in virtual
// pages (gw_plan.h: the two partial pages at the ends of a full window are
// walked as one, so a 1024-token window is 64 pages of work: 2 splits of 32
// at group size 1 or 2, 4 of 16 at group size 4).  The W waves of a
// workgroup (8, or 4 at group size 4) take every W-th page of the split, 4
// pages each on a full window, each wave with its own online softmax state
// (running max m, sum l, accumulator), merged in LDS at the end.
// The last workgroup of a (sequence, KV head) to finish merges the splits'
// partials in split order (a counter per pair, reset by that workgroup).
//
// Lane roles inside a wave (the page layout puts each lane's 16 bytes next
// to its neighbours', so every load instruction reads a contiguous 1 KiB):
//   QK: lane = 4*t + c holds 64 dims (c-th quarter) of token t of the page;
//       q.K is a chain of v_dot2_f32_bf16 over the quarter, then a 4-lane
//       DPP sum -- one 16-token page per wave instruction group.
//   PV: lane l owns output dims 4l..4l+3 and holds V as (token, token+1)
//       bf16 pairs per dim, so acc += dot2(V pair, P pair) with the P pairs
//       broadcast from SGPRs; no cross-lane reduction over tokens at all.
// P is rounded to bf16 for PV and the sum l adds exactly those rounded
// values, so the normalisation matches the weights used.
// e4m3 pages hold the same roles at one byte per element; two codes convert
// to a bf16 pair exactly (v_cvt_scalef32_pk_bf16_fp8, scale 1).

#include "gw_device.h"
#include "gw_kernels.h"
#include "gw_plan.h"
#include "gw_rows_append.h"

namespace gw {
namespace {

constexpr int kLocalD = 256;
// Page-table rows up to this many entries are read whole into LDS.
constexpr int kLocalPtLds = 2048;
// Re-reads of one partial before the reducing workgroup gives up on it.
constexpr int kLocalMaxReReads = 1 << 20;

template <bool FP8>
struct LocalLayout {
  static constexpr int kBlockBytes = FP8 ? 4096 : 8192;  // one K or V block of a page
  static constexpr int kLoads = FP8 ? 4 : 8;             // 16-byte loads per block per lane
};

template <bool FP8>
struct PageRegs {
  uint4 k[LocalLayout<FP8>::kLoads];
  uint4 v[LocalLayout<FP8>::kLoads];
  uint4 vx;   // merged page: the V unit that straddles the two pages, from the first page
};

// Load one virtual page: slots t >= b from the (page, KV head) record r0,
// slots t < b from r1 (r1 == r0 and b == 0 for an ordinary page).  K lane
// 4t + c takes token t, so the choice is per lane; a V load u holds the
// tokens of one pair (bf16) or quad (e4m3), so it is per instruction, and
// the unit holding slots on both sides of b is loaded from both records.
template <bool FP8>
__device__ __forceinline__ void load_vpage(PageRegs<FP8>& r, const uint8_t* r0, const uint8_t* r1, int b,
                                           int lane) {
  constexpr int kTok = FP8 ? 4 : 2;   // tokens per V unit
  const uint8_t* kb = ((lane >> 2) >= b ? r0 : r1) + lane * 16;
#pragma unroll
  for (int k = 0; k < LocalLayout<FP8>::kLoads; ++k) r.k[k] = ld16(kb + k * 1024);
#pragma unroll
  for (int u = 0; u < LocalLayout<FP8>::kLoads; ++u)
    r.v[u] = ld16((kTok * u >= b ? r0 : r1) + LocalLayout<FP8>::kBlockBytes + u * 1024 + lane * 16);
  if (b % kTok != 0)
    r.vx = ld16(r0 + LocalLayout<FP8>::kBlockBytes + (b / kTok) * 1024 + lane * 16);
}

// A page table (or other int32 array) read-only for the whole call, read
// through the constant address space so uniform reads become scalar loads.
typedef const __attribute__((address_space(4))) int32_t* CI32P;

// One virtual page of a wave's walk (load_vpage / process_page arguments).
struct VPage {
  const uint8_t* r0;
  const uint8_t* r1;
  int b;
  uint32_t mask;
};

__device__ __forceinline__ uint32_t u4_get(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ __forceinline__ void u4_set(uint4& v, int i, uint32_t x) {
  if (i == 0) v.x = x; else if (i == 1) v.y = x; else if (i == 2) v.z = x; else v.w = x;
}
__device__ __forceinline__ void u4_and(uint4& v, uint32_t m) {
  v.x &= m; v.y &= m; v.z &= m; v.w &= m;
}

// The new token of a decode row: lane l loads K dims 4l..4l+3 with their
// rotation partners 128 + 4l.. and the rotary factors (lanes < 32), and V
// dims 4l..4l+3 (every lane), before the page itself, so the two overlap.
struct NewTokenLoads {
  uint2 kr, kp, v;
  float4 cs, sn;
};

__device__ __forceinline__ NewTokenLoads load_new_token(const LocalAttnArgs& a, int row, int g, int p, int lane) {
  NewTokenLoads t{};
  const int64_t src = ((int64_t)row * a.num_kv_heads + g) * kLocalD;
  if (lane < 32) {
    t.kr = *reinterpret_cast<const uint2*>(a.k_new + src + 4 * lane);
    t.kp = *reinterpret_cast<const uint2*>(a.k_new + src + 128 + 4 * lane);
    if (a.rope_cos) {
      t.cs = *reinterpret_cast<const float4*>(a.rope_cos + (int64_t)p * 128 + 4 * lane);
      t.sn = *reinterpret_cast<const float4*>(a.rope_sin + (int64_t)p * 128 + 4 * lane);
    }
  }
  t.v = *reinterpret_cast<const uint2*>(a.v_new + src + 4 * lane);
  return t;
}

// Rotate and round the new token's K and store K and V into the pool (b:
// the (page, KV head) record) element by element, exactly as gw_kv_append
// does; then put the token into this wave's registers of that page: K
// through the wave's own 1 KiB of LDS (sm_tok), V straight from the lane's
// own dims.
template <bool FP8>
__device__ __forceinline__ void put_new_token(PageRegs<FP8>& r, uint8_t* b, const NewTokenLoads& t, bool rope,
                                              int p, int lane, uint32_t* sm_tok) {
  const int slot = p & 15;
  if (lane < 32) {
    float xa[4] = {bf16_lo(t.kr.x), bf16_hi(t.kr.x), bf16_lo(t.kr.y), bf16_hi(t.kr.y)};
    float xb[4] = {bf16_lo(t.kp.x), bf16_hi(t.kp.x), bf16_lo(t.kp.y), bf16_hi(t.kp.y)};
    float ya[4], yb[4];
    const float c4[4] = {t.cs.x, t.cs.y, t.cs.z, t.cs.w}, s4[4] = {t.sn.x, t.sn.y, t.sn.z, t.sn.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (rope) rope_pair(xa[j], xb[j], c4[j], s4[j], ya[j], yb[j]);
      else { ya[j] = xa[j]; yb[j] = xb[j]; }
    }
    // dims d = 4l..4l+3 (quarter c = l/16) and d + 128 (quarter c + 2)
    const int c = lane >> 4;
    if constexpr (!FP8) {
      const int k = (lane & 15) >> 1, e0 = 4 * (lane & 1);
      uint16_t* kb = reinterpret_cast<uint16_t*>(b);
      const uint2 va = {pack_bf16(ya[0], ya[1]), pack_bf16(ya[2], ya[3])};
      const uint2 vb = {pack_bf16(yb[0], yb[1]), pack_bf16(yb[2], yb[3])};
      *reinterpret_cast<uint2*>(kb + ((k * 16 + slot) * 4 + c) * 8 + e0) = va;
      *reinterpret_cast<uint2*>(kb + ((k * 16 + slot) * 4 + c + 2) * 8 + e0) = vb;
      sm_tok[2 * lane] = va.x;
      sm_tok[2 * lane + 1] = va.y;
      sm_tok[64 + 2 * lane] = vb.x;
      sm_tok[64 + 2 * lane + 1] = vb.y;
    } else {
      const int k = (lane & 15) >> 2, e0 = 4 * (lane & 3);
      uint32_t wa = 0, wb = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wa |= f32_to_e4m3(round_bf16(ya[j])) << (8 * j);
        wb |= f32_to_e4m3(round_bf16(yb[j])) << (8 * j);
      }
      *reinterpret_cast<uint32_t*>(b + ((k * 16 + slot) * 4 + c) * 16 + e0) = wa;
      *reinterpret_cast<uint32_t*>(b + ((k * 16 + slot) * 4 + c + 2) * 16 + e0) = wb;
      sm_tok[lane] = wa;
      sm_tok[32 + lane] = wb;
    }
  }
  // V: dims 4l + j of token slot -> interleaved pairs (bf16) or quads (e4m3)
  const uint32_t v16[4] = {t.v.x & 0xffffu, t.v.x >> 16, t.v.y & 0xffffu, t.v.y >> 16};
  uint32_t bits[4];
  if constexpr (!FP8) {
    uint16_t* vb = reinterpret_cast<uint16_t*>(b + LocalLayout<FP8>::kBlockBytes);
    const int u = slot >> 1, i = slot & 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vb[((u * 64 + lane) * 4 + j) * 2 + i] = (uint16_t)v16[j];
      bits[j] = v16[j];
    }
  } else {
    uint8_t* vb = b + LocalLayout<FP8>::kBlockBytes;
    const int u = slot >> 2, i = slot & 3;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bits[j] = f32_to_e4m3(bits_to_f32(v16[j] << 16));
      vb[((u * 64 + lane) * 4 + j) * 4 + i] = (uint8_t)bits[j];
    }
  }
  // registers: V of the token's slot in this lane's pair / quad registers
  constexpr int kTokPerReg = FP8 ? 4 : 2;
  const int u = slot / kTokPerReg;
  const int sh = (FP8 ? 8 : 16) * (slot % kTokPerReg);
  const uint32_t field = (FP8 ? 0xffu : 0xffffu) << sh;
#pragma unroll
  for (int uu = 0; uu < LocalLayout<FP8>::kLoads; ++uu) {
    const uint32_t m = (uu == u) ? field : 0u;
    r.v[uu].x = (r.v[uu].x & ~m) | ((bits[0] << sh) & m);
    r.v[uu].y = (r.v[uu].y & ~m) | ((bits[1] << sh) & m);
    r.v[uu].z = (r.v[uu].z & ~m) | ((bits[2] << sh) & m);
    r.v[uu].w = (r.v[uu].w & ~m) | ((bits[3] << sh) & m);
  }
  // K of the token's slot: lane (t = slot, c) holds dims 64c + kPer k .. of
  // register k (kPer = 8 bf16 / 16 e4m3 per 16 bytes)
  if ((lane >> 2) == slot) {
    const int c = lane & 3;
#pragma unroll
    for (int k = 0; k < LocalLayout<FP8>::kLoads; ++k) {
      const int w0 = FP8 ? 16 * c + 4 * k : 32 * c + 4 * k;   // first 32-bit word of the chunk
      r.k[k] = uint4{sm_tok[w0], sm_tok[w0 + 1], sm_tok[w0 + 2], sm_tok[w0 + 3]};
    }
  }
}

// The group's q in LDS: head h's 16-byte chunk j (dims 8j .. 8j + 7, bf16
// pairs) at chunk h * 32 + (j ^ ((j / 8) % 8)); the four quarters a lane
// reads together (chunks 8c + k, c = 0..3) sit in distinct banks, and every
// lane of a quad reads the same chunk.
typedef __attribute__((address_space(3))) const u32x4 lds_q4;

// One virtual page: b as in load_vpage, mask = its slots inside the row's
// range (bit t for slot t; 0xffff for every page but the range's edges).
// q: bf16 pages take it from registers (qr, the lane's quarter of each head),
// e4m3 pages from LDS (qh: the K codes widen once for every head of the
// group, and the registers q would take are left to the page buffers).
template <int G, bool FP8>
__device__ __forceinline__ void process_page(PageRegs<FP8>& r, const uint32_t (&qr)[G][32], lds_q4* qh,
                                             uint32_t mask, int b, float scale_log2, int lane,
                                             float (&m_run)[G], float (&l_run)[G],
                                             float (&acc)[G][4]) {
  const int t = lane >> 2;
  constexpr int kTok = FP8 ? 4 : 2;
  if (b % kTok != 0) {
    // the V unit holding slots b - 1 and b: slots >= b come from the first page
    const uint32_t keep = FP8 ? (1u << (8 * (b % 4))) - 1u : 0x0000ffffu;
    // as masks on every unit (a branch per unit would select a register by
    // a run-time index, which the compiler may place in scratch)
#pragma unroll
    for (int u = 0; u < LocalLayout<FP8>::kLoads; ++u) {
      const uint32_t take = u == b / kTok ? ~keep : 0u;
      r.v[u].x = (r.v[u].x & ~take) | (r.vx.x & take);
      r.v[u].y = (r.v[u].y & ~take) | (r.vx.y & take);
      r.v[u].z = (r.v[u].z & ~take) | (r.vx.z & take);
      r.v[u].w = (r.v[u].w & ~take) | (r.vx.w & take);
    }
  }
  // ---- scores: lane (t, c) dots its quarter of K_t with q, then quad sum;
  // per head the products go into two chains in the order k, m
  float s0[G], s1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) s0[h] = s1[h] = 0.f;
  if constexpr (!FP8) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float& s = (k & 1) ? s1[h] : s0[h];
#pragma unroll
        for (int m = 0; m < 4; ++m) s = dot2_bf16(u4_get(r.k[k], m), qr[h][4 * k + m], s);
      }
    }
  } else {
    const int c = lane & 3;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // the K codes widen to bf16 once, for every head of the group
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t w = u4_get(r.k[k], m);
        lo[m] = e4m3x2_to_bf16x2<false>(w);
        hi[m] = e4m3x2_to_bf16x2<true>(w);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float& s = (k & 1) ? s1[h] : s0[h];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int j = 8 * c + 2 * k + half;
          const u32x4 qv = qh[h * 32 + (j ^ ((j >> 3) & 7))];
          s = dot2_bf16(lo[2 * half], qv[0], s);
          s = dot2_bf16(hi[2 * half], qv[1], s);
          s = dot2_bf16(lo[2 * half + 1], qv[2], s);
          s = dot2_bf16(hi[2 * half + 1], qv[3], s);
        }
      }
    }
  }
  float z[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float s = s0[h] + s1[h];
    s += dpp_f32<kQuadSwap1>(s);
    s += dpp_f32<kQuadSwap2>(s);
    z[h] = s;
  }
  const bool valid = (mask >> t) & 1u;
#pragma unroll
  for (int h = 0; h < G; ++h) z[h] = valid ? z[h] * scale_log2 : -INFINITY;

  // ---- online softmax: page max, rescale on a new maximum (wave-uniform)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mx = wave_max_quads(z[h]);
    const float mnew = fmaxf(m_run[h], mx);
    if (mnew > m_run[h]) {
      const float alpha = __builtin_amdgcn_exp2f(m_run[h] - mnew);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[h][j] *= alpha;
      l_run[h] *= alpha;
      m_run[h] = mnew;
    }
  }

  // ---- probabilities, rounded to bf16 pairs (token 2u, 2u+1) in SGPRs
  uint32_t P[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float pr = __builtin_amdgcn_exp2f(z[h] - m_run[h]);  // 0 where masked
    const float nb = dpp_f32<kRowShl4>(pr);                      // token t + 1
    const uint32_t pair = pack_bf16(pr, nb);
    l_run[h] += bf16_lo(pair);
#pragma unroll
    for (int u = 0; u < 8; ++u) P[h][u] = readlane_u32(pair, 8 * u);
  }

  // ---- V of masked slots (the range's edge pages only) is zeroed, so that
  // unwritten or stale slots (possibly NaN) contribute exactly 0.
  if (mask != 0xffffu) {
    if constexpr (!FP8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t m = (((mask >> (2 * u)) & 1u) ? 0x0000ffffu : 0u) |
                           (((mask >> (2 * u + 1)) & 1u) ? 0xffff0000u : 0u);
        u4_and(r.v[u], m);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((mask >> (4 * u + i)) & 1u) m |= 0xffu << (8 * i);
        u4_and(r.v[u], m);
      }
    }
  }

  // ---- PV: lane owns dims 4l..4l+3
  if constexpr (!FP8) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[h][j] = dot2_bf16(u4_get(r.v[u], j), P[h][u], acc[h][j]);
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = u4_get(r.v[u], j);
        const uint32_t lo2 = e4m3x2_to_bf16x2<false>(w);   // tokens 4u, 4u+1
        const uint32_t hi2 = e4m3x2_to_bf16x2<true>(w);    // tokens 4u+2, 4u+3
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][j] = dot2_bf16(lo2, P[h][2 * u], acc[h][j]);
          acc[h][j] = dot2_bf16(hi2, P[h][2 * u + 1], acc[h][j]);
        }
      }
  }
}

// The reducing workgroup's merge of q heads h0 .. h0 + GH - 1, output dim d:
// every split's (max, sum, acc) is loaded at once (all of them again while
// any pair's tag is not yet this call's), then M = max_i m_i,
// l = sum_i l_i 2^(m_i - M), out = sum_i acc_i 2^(m_i - M) / l, both sums
// in split order.  NS bounds nsplit.  Returns false, after writing NaN, if a
// pair never arrived.
template <int GH, int NS>
__device__ __forceinline__ bool merge_splits(const LocalAttnArgs& a, int s, int h0, int row, int d, int nsplit,
                                             uint64_t tag) {
  uint64_t mi[GH][NS], li[GH][NS], ai[GH][NS];
  // one copy of the load code (the kernel's tail runs from a cold
  // instruction cache): read everything, and again while any pair is stale.
  // The first read is a plain one: the splits of a (sequence, KV head) are
  // dispatched (KV heads x sequences) workgroups apart, a multiple of the 8
  // XCDs that workgroups are dealt to in turn when the KV heads number 8, so
  // they share an XCD and its L2, which the writers' stores pass through.  Wherever the
  // workgroups ran, a pair read from a stale line carries an old tag and is
  // read again at device scope, so the result never depends on placement.
  bool ok = true;
  for (int spin = 0;; ++spin) {
    bool all = true;
#pragma unroll
    for (int h = 0; h < GH; ++h)
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        mi[h][i] = li[h][i] = ai[h][i] = tag;
        if (i < nsplit) {
          const int64_t ic = ((int64_t)s * a.num_q_heads + h0 + h) * a.max_splits + i;
          if (spin == 0) {   // may be served by this XCD's L2
            mi[h][i] = __hip_atomic_load(a.part_ml + ic * 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            li[h][i] = __hip_atomic_load(a.part_ml + ic * 2 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            ai[h][i] = __hip_atomic_load(a.part_acc + ic * kLocalD + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          } else {           // from the memory side
            mi[h][i] = __hip_atomic_load(a.part_ml + ic * 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            li[h][i] = __hip_atomic_load(a.part_ml + ic * 2 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ai[h][i] = __hip_atomic_load(a.part_acc + ic * kLocalD + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
#pragma unroll
    for (int h = 0; h < GH; ++h)
#pragma unroll
      for (int i = 0; i < NS; ++i)
        all &= ((mi[h][i] >> 32) == (tag >> 32)) & ((li[h][i] >> 32) == (tag >> 32)) & ((ai[h][i] >> 32) == (tag >> 32));
    if (all) break;
    if (spin == kLocalMaxReReads) { ok = false; break; }
  }
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    float Mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (i < nsplit) Mx = fmaxf(Mx, bits_to_f32((uint32_t)mi[h][i]));
    float ls = 0.f, ov = 0.f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i < nsplit) {
        const float sw = __builtin_amdgcn_exp2f(bits_to_f32((uint32_t)mi[h][i]) - Mx);
        ls += bits_to_f32((uint32_t)li[h][i]) * sw;
        ov += bits_to_f32((uint32_t)ai[h][i]) * sw;
      }
    }
    a.out[((int64_t)row * a.num_q_heads + h0 + h) * kLocalD + d] = ok ? ov / ls : __builtin_nanf("");
  }
  return ok;
}

// A split index of the workgroup's range as a type (its value known at
// compile time, so per-split state stays in registers).
template <int J>
struct SplitIndex {
  static constexpr int value = J;
};
// a or b, chosen at compile time (a run-time choice of a reference would
// make both addressable and move them to scratch)
template <bool FIRST, class T>
__device__ __forceinline__ T& pick(T& a, T& b) {
  if constexpr (FIRST) return a;
  else return b;
}

// SPW: consecutive splits of a (sequence, KV head) taken by one workgroup
// (1, 2 or 4; the host picks it from the batch).  The plan, the pages each
// wave walks for a split and the order it walks them, and every merge are
// those of one split per workgroup, so results do not depend on SPW.
template <int G, bool FP8, int SPW>
__global__ __launch_bounds__(64 * local_waves(G), 1) void local_decode_kernel(LocalAttnArgs a) {
  constexpr int kLocalWaves = local_waves(G);
  constexpr int kLocalThreads = 64 * kLocalWaves;
  const int tid = threadIdx.x, lane = tid & 63;
  // trace slots: 0 XCD | split << 8 | KV head << 16 | sequence << 32,
  // 1 pages of wave 0 | splits << 16 | merged << 32, 2 entry, 3 q and page
  // table in LDS, 4 wave 0's pages done, 5 waves merged, 6 arrival counted,
  // 7 exit, 8 + w wave w's pages done
  GW_TRACE_T(a, 2, tid == 0);
  // the workgroups past the decode items append the prompt rows' own
  // tokens, 256 threads a unit (the prompt rows attend in the next launch)
  if ((int)blockIdx.x >= a.append_wg0) {
    local_rows_append_unit<FP8>(a, ((int)blockIdx.x - a.append_wg0) * (kLocalThreads / 256) + tid / 256, tid % 256);
    return;
  }
  const int w = uniform_i32(tid >> 6);
  // Workgroups go split-major (every pair's split 0, then every pair's
  // split 1, ...), rows fastest: a pair's splits are dispatched apart, which
  // measures faster than dispatching them side by side.  With one row per
  // sequence the sequences are the rows; with q_indptr the decode sequences
  // (one row each; prompt rows go elsewhere) are numbered compactly, in
  // order, so that the workgroups the grid holds for the prompt sequences
  // come last and leave, instead of holding CUs ahead of working ones.
  int split, g, s, row;   // split: the first of the workgroup's SPW splits
  if (a.q_indptr == nullptr) {
    const int npairs = a.num_kv_heads * a.num_seqs;
    split = (int)blockIdx.x / npairs * SPW;
    const int rem = (int)blockIdx.x % npairs;
    g = rem / a.num_seqs;
    s = row = rem % a.num_seqs;
  } else {
    // the decode sequences of 64-sequence chunk c0, as a lane mask, and
    // the rows where each lane's sequence starts
    auto chunk = [&](int c0, int& r0) __attribute__((always_inline)) {
      const int sl = c0 + lane;
      r0 = sl < a.num_seqs ? a.q_indptr[sl] : 0;
      return (uint64_t)__ballot(sl < a.num_seqs && a.q_indptr[sl + 1] - r0 == 1);
    };
    int r0 = 0;
    uint64_t m = chunk(0, r0);
    int n_dec = __popcll(m);
    for (int c0 = 64; c0 < a.num_seqs; c0 += 64) {
      int r1;
      n_dec += __popcll(chunk(c0, r1));
    }
    const int ndp = a.num_kv_heads * n_dec;
    if (ndp == 0 || (int)blockIdx.x >= cdiv_i(a.max_splits, SPW) * ndp) return;
    split = (int)blockIdx.x / ndp * SPW;
    const int rem = (int)blockIdx.x % ndp;
    g = rem / n_dec;
    int k = rem % n_dec;   // rank of the sequence among the decode sequences
    int c0 = 0;
    while (k >= __popcll(m)) {   // ends: k < n_dec, the total count
      k -= __popcll(m);
      c0 += 64;
      m = chunk(c0, r0);
    }
    const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    const int ls = __builtin_ctzll(__ballot(((m >> lane) & 1) && rank == k));
    s = c0 + ls;
    row = __builtin_amdgcn_readlane(r0, ls);
  }
  split = uniform_i32(split);
  g = uniform_i32(g);
  s = uniform_i32(s);
  row = uniform_i32(row);

  // The page-table row (when it has at most kLocalPtLds entries) and the
  // group's q are read in the same round trip as the sequence's length --
  // before it is known which pages the window covers -- and go to LDS.
  const auto q_chunk = [&](int r) __attribute__((always_inline)) {   // chunk tid % 32 of head tid / 32
    return *reinterpret_cast<const u32x4*>(a.q + ((int64_t)r * a.num_q_heads + g * G + tid / 32) * kLocalD +
                                           8 * (tid % 32));
  };
  u32x4 qv = {0u, 0u, 0u, 0u};
  if (tid < 32 * G) qv = q_chunk(row);
  const int L = ((CI32P)a.seq_lens)[s];
  const bool pt_lds = a.pt_stride <= kLocalPtLds;
  int ptv[kLocalPtLds / kLocalThreads] = {};
  if (pt_lds) {
    const int32_t* prow = a.page_table + (int64_t)s * a.pt_stride;
#pragma unroll
    for (int i = 0; i < kLocalPtLds / kLocalThreads; ++i)
      if (tid + kLocalThreads * i < a.pt_stride) ptv[i] = prow[tid + kLocalThreads * i];
  }
  const int p = L - 1;
  const LocalWindow win = local_window(p, a.window);
  const int nsplit = local_nsplit(win.nv, G);
  if (split >= nsplit) return;
  const int n_own = min(SPW, nsplit - split);   // splits split .. split + n_own - 1
  // the whole row's range in this workgroup: its splits merge in registers
  const bool covers_all = split == 0 && n_own == nsplit;
  int v0s[SPW], v1s[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    v0s[j] = j < n_own ? split_lo(win.nv, nsplit, split + j) : 0;
    v1s[j] = j < n_own ? split_lo(win.nv, nsplit, split + j + 1) : 0;
  }
  const int v0 = v0s[0], v1 = v1s[0];
  const int v_end = SPW == 1 ? v1 : split_lo(win.nv, nsplit, split + n_own);
  // the virtual page holding position p, where a decode row's new token goes
  const int vt = win.wrap ? 0 : win.nv - 1;
  const bool token_here = vt >= v0 && vt < v_end;
  const bool append_here = a.v_new != nullptr && token_here;

  // q chunk j of a head sits at chunk j ^ ((j / 8) % 8) in LDS, so that the
  // four quarters read below (chunks 8c + k, c = 0..3) hit distinct banks
  __shared__ int sm_pt[kLocalPtLds];
  __shared__ __attribute__((aligned(16))) uint32_t sm_q[G][128];
  if (pt_lds) {
#pragma unroll
    for (int i = 0; i < kLocalPtLds / kLocalThreads; ++i)
      if (tid + kLocalThreads * i < a.pt_stride) sm_pt[tid + kLocalThreads * i] = ptv[i];
  }
  if (tid < 32 * G) {
    const int j = tid % 32;
    *reinterpret_cast<u32x4*>(&sm_q[tid / 32][4 * (j ^ ((j >> 3) & 7))]) = qv;
  }
  __syncthreads();
  GW_TRACE_T(a, 3, tid == 0);
  GW_TRACE_V(a, 0, tid == 0, GW_TRACE_XCC() | (uint64_t)split << 8 | (uint64_t)g << 16 | (uint64_t)s << 32);

  // q of the group, this lane's quarter of the dims, as bf16 pairs (bf16
  // pages; e4m3 pages read it from LDS)
  const int c = lane & 3;
  uint32_t qr[G][32];
  lds_q4* qh = (lds_q4*)&sm_q[0][0];
#pragma unroll
  for (int h = 0; h < (FP8 ? 0 : G); ++h) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = 8 * c + k;
      const u32x4 v = *reinterpret_cast<const u32x4*>(&sm_q[h][4 * (j ^ ((j >> 3) & 7))]);
      qr[h][4 * k + 0] = v[0]; qr[h][4 * k + 1] = v[1];
      qr[h][4 * k + 2] = v[2]; qr[h][4 * k + 3] = v[3];
    }
  }

  float m_run[G], l_run[G], acc[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[h][j] = 0.f;
  }

  // This wave's pages are virtual pages v0 + w + 4k, k < nw.  The wave
  // holding the token's page takes it first and the rest in order; every
  // other wave goes in order.  The order is the same whether or not the call
  // appends, so results are too.  Page ids come from the LDS copy of the
  // row, or, for longer rows, from scalar loads (the page table is read-only
  // during the call) issued a page ahead of their use.
  const int nw = (v1 - v0 - w + kLocalWaves - 1) / kLocalWaves;
  const bool tok_wave = token_here && w == (vt - v0) % kLocalWaves;
  const int k_tok = tok_wave ? (vt - v0) / kLocalWaves : 0;
  auto k_of = [&](int i) __attribute__((always_inline)) {
    return !tok_wave ? i : i == 0 ? k_tok : (i <= k_tok ? i - 1 : i);
  };
  const CI32P pt = (CI32P)(a.page_table + (int64_t)s * a.pt_stride);
  const uint8_t* head_base = a.pool + (int64_t)g * a.head_bytes;
  const int mlo = win.lo & 15, mhi = p & 15;
  auto vpage_at = [&](int vbase, int k) __attribute__((always_inline)) {
    const int v = vbase + w + kLocalWaves * k;
    const bool merged = win.wrap && v == 0;
    const int id0 = pt_lds ? uniform_i32(sm_pt[win.pg0 + v]) : pt[win.pg0 + v];
    const int id1 = merged ? (pt_lds ? uniform_i32(sm_pt[win.pgl]) : pt[win.pgl]) : id0;
    VPage d;
    d.r0 = head_base + (int64_t)id0 * a.page_bytes;
    d.r1 = head_base + (int64_t)id1 * a.page_bytes;
    d.b = merged ? win.b : 0;
    uint32_t m = 0xffffu;
    if (merged) {
      m = (0xffffu << mlo) | ((2u << mhi) - 1u);
    } else if (!win.wrap) {
      if (v == 0) m &= 0xffffu << mlo;
      if (v == win.nv - 1) m &= (2u << mhi) - 1u;
    }
    d.mask = m & 0xffffu;
    return d;
  };
  auto vpage = [&](int k) __attribute__((always_inline)) { return vpage_at(v0, k); };

  // this (sequence, KV head)'s call count, the tag of this call's partials:
  // read behind the first page's loads (a device-scope load goes to memory,
  // and any wait for it would hold the page requests back), first used after
  // the page loop (the empty asm there keeps the compiler from waiting for
  // it earlier)
  uint32_t epoch = 0u;
  auto load_epoch = [&]() __attribute__((always_inline)) {
    return __hip_atomic_load(a.epochs + (int64_t)s * a.num_kv_heads + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  __shared__ uint32_t sm_tok[kLocalWaves][128];   // a patching wave's rotated token K
  if constexpr (SPW == 1) {
  // One page buffer per wave: a page's loads are issued as soon as the page
  // before it has been processed, so a wave has one page in flight while it
  // waits and none while it computes.  Two or three buffers per wave (the
  // next pages loading while one is processed) measured slower: the CU's
  // eight waves keep enough in flight, and more queued transfers only
  // lengthen each one's wait.
  PageRegs<FP8> A;
  VPage dA{}, dn{};   // this page's descriptor, the next page's
  if (nw > 0) {
    const bool patch = append_here && tok_wave;
    NewTokenLoads tok{};
    if (patch) tok = load_new_token(a, row, g, p, lane);
    dA = vpage(k_of(0));
    load_vpage<FP8>(A, dA.r0, dA.r1, dA.b, lane);
    if (nw > 1) dn = vpage(k_of(1));
    if (patch) {
      const int id_tok = pt_lds ? uniform_i32(sm_pt[win.pgl]) : pt[win.pgl];
      uint8_t* rec = const_cast<uint8_t*>(head_base) + (int64_t)id_tok * a.page_bytes;
      put_new_token<FP8>(A, rec, tok, a.rope_cos != nullptr, p, lane, sm_tok[w]);
    }
  }
  if (nsplit > 1) epoch = load_epoch();
  for (int j = 0; j < nw; ++j) {
    process_page<G, FP8>(A, qr, qh, dA.mask, dA.b, a.scale_log2, lane, m_run, l_run, acc);
    if (j + 1 < nw) {
      dA = dn;
      load_vpage<FP8>(A, dA.r0, dA.r1, dA.b, lane);
      if (j + 2 < nw) dn = vpage(k_of(j + 2));
    }
  }

  asm volatile("" : "+v"(epoch));
  GW_TRACE_T(a, 4, tid == 0);
  GW_TRACE_T(a, 8 + w, lane == 0);
  GW_TRACE_V(a, 1, tid == 0, (uint64_t)nw | (uint64_t)nsplit << 16);
  // ---- merge the waves in LDS, in wave order
  __shared__ float sm_acc[kLocalWaves][G][kLocalD];
  __shared__ float sm_m[kLocalWaves][G], sm_l[kLocalWaves][G];
  __shared__ int sm_last;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float lv = (c == 0) ? l_run[h] : 0.f;   // one lane per token slot
    lv += shfl_xor_f32(lv, 4);
    lv += shfl_xor_f32(lv, 8);
    lv += shfl_xor_f32(lv, 16);
    lv += shfl_xor_f32(lv, 32);
    if (lane == 0) {
      sm_m[w][h] = m_run[h];
      sm_l[w][h] = lv;
    }
    *reinterpret_cast<f32x4*>(&sm_acc[w][h][4 * lane]) = f32x4{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
  }
  __syncthreads();

  // the first 256 threads take one output dim each; with 8 waves the others
  // mirror dim 0, write nothing, and only meet the barriers
  const bool dt = tid < kLocalD;
  const int d = dt ? tid : 0;
  float o[G], M[G], lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    M[h] = sm_m[0][h];
#pragma unroll
    for (int ww = 1; ww < kLocalWaves; ++ww) M[h] = fmaxf(M[h], sm_m[ww][h]);
    lsum[h] = 0.f;
    o[h] = 0.f;
#pragma unroll
    for (int ww = 0; ww < kLocalWaves; ++ww) {
      const float mw = sm_m[ww][h];
      const float sw = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M[h]);
      lsum[h] += sm_l[ww][h] * sw;
      o[h] += sm_acc[ww][h][d] * sw;
    }
  }
  GW_TRACE_T(a, 5, tid == 0);
  if (nsplit == 1) {
    if (!dt) return;
#pragma unroll
    for (int h = 0; h < G; ++h)
      a.out[((int64_t)row * a.num_q_heads + g * G + h) * kLocalD + d] = o[h] / lsum[h];
    GW_TRACE_T(a, 7, tid == 0);
    return;
  }

  // ---- publish this split's partial; the last workgroup of the (sequence,
  // KV head) to arrive reduces all of them in split order.  Every value goes
  // out as one 64-bit (value, tag) pair, tag = this call's epoch, with
  // device-scope atomic stores, and the arrival counter moves right after
  // the stores are issued, without waiting for them: the last workgroup
  // reads each pair (atomic 64-bit loads: plain first, then device scope)
  // and reads again, until its tag is this call's, the few pairs whose
  // stores are still on their way.  Every pair it waits for was stored before its writer's arrival,
  // so each wait ends; a bound on the re-reads turns a broken invariant
  // into NaN output instead of a hang.
  const uint64_t tag = (uint64_t)(epoch + 1u) << 32;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (!dt) break;
    const int64_t pi = ((int64_t)s * a.num_q_heads + g * G + h) * a.max_splits + split;
    __hip_atomic_store(a.part_acc + pi * kLocalD + d, tag | f32_to_bits(o[h]), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (d == 0) {
      __hip_atomic_store(a.part_ml + pi * 2 + 0, tag | f32_to_bits(M[h]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.part_ml + pi * 2 + 1, tag | f32_to_bits(lsum[h]), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Every store of the workgroup is issued, not waited for: the barriers
  // here order LDS only (a full __syncthreads would wait for the stores).
  lds_barrier();
  int* counter = a.counters + (int64_t)s * a.num_kv_heads + g;
  if (tid == 0)
    sm_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nsplit - 1;
  lds_barrier();
  GW_TRACE_T(a, 6, tid == 0);
  if (!sm_last || !dt) {
    GW_TRACE_T(a, 7, tid == 0);
    return;
  }
  // The heads of the group are merged together, so their loads share one
  // round trip; a row's range of up to 68 pages has at most 4 splits (at
  // either split size).
  bool ok;
  if (nsplit <= 4) {
    ok = merge_splits<G, 4>(a, s, g * G, row, d, nsplit, tag);
  } else {
    ok = true;
#pragma unroll
    for (int h = 0; h < G; ++h) ok &= merge_splits<1, kLocalMaxSplits>(a, s, g * G + h, row, d, nsplit, tag);
  }
  (void)ok;
  if (tid == 0) {   // ready for the next call
    __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.epochs + (int64_t)s * a.num_kv_heads + g, epoch + 1u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  GW_TRACE_V(a, 1, tid == 0, (uint64_t)nw | (uint64_t)nsplit << 16 | 1ull << 32);
  GW_TRACE_T(a, 7, tid == 0);
  } else {
    // ---- SPW splits per workgroup.  Wave w walks, for each split j, the
    // same pages in the same order as the workgroup of that split alone
    // would (virtual pages v0_j + w + W k; the token's page first on the
    // wave that holds it), into a softmax state of that split's own.  The
    // walk interleaves the splits page by page, items (i, j) in that order,
    // with item (i, j) in buffer A (j even) or B (j odd), so the next item
    // always loads into the other buffer while this one is processed.  An
    // item past a split's pages (or of a split past the row's last) is
    // processed as a page with no slot in range: no load, nothing added.
    static_assert(SPW == 2 || SPW == 4, "items alternate between the two buffers");
    float m_s[SPW][G], l_s[SPW][G], acc_s[SPW][G][4];
#pragma unroll
    for (int j = 0; j < SPW; ++j)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        m_s[j][h] = -INFINITY;
        l_s[j][h] = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc_s[j][h][e] = 0.f;
      }
    int nws[SPW];
    int nw_max = 0;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      nws[j] = j < n_own ? max(0, (v1s[j] - v0s[j] - w + kLocalWaves - 1) / kLocalWaves) : 0;
      nw_max = max(nw_max, nws[j]);
    }
    int j_tok = 0;
#pragma unroll
    for (int j = 1; j < SPW; ++j)
      if (j < n_own && vt >= v0s[j]) j_tok = j;
    int v0_tok = v0s[0];
#pragma unroll
    for (int j = 1; j < SPW; ++j)
      if (j == j_tok) v0_tok = v0s[j];
    const bool tok_w = token_here && w == (vt - v0_tok) % kLocalWaves;
    const int k_tk = tok_w ? (vt - v0_tok) / kLocalWaves : 0;
    auto k_at = [&](int j, int i) __attribute__((always_inline)) {
      return (!tok_w || j != j_tok) ? i : i == 0 ? k_tk : (i <= k_tk ? i - 1 : i);
    };
    auto real = [&](int j, int i) __attribute__((always_inline)) { return i < nws[j]; };
    const bool patch = append_here && tok_w;
    NewTokenLoads tok{};
    if (patch) tok = load_new_token(a, row, g, p, lane);
    // bf16 pages: two buffers, the next item loading while one is processed;
    // e4m3 pages: one buffer, loaded once the item before it is processed
    // (faster for e4m3 at 64 x 8192, slower for bf16 at group size 4)
    constexpr bool kOneBuf = FP8;
    PageRegs<FP8> A, B;
    VPage dA{}, dB{};
    if (real(0, 0)) {
      dA = vpage_at(v0s[0], k_at(0, 0));
      load_vpage<FP8>(A, dA.r0, dA.r1, dA.b, lane);
    }
    if (nsplit > 1 && !covers_all) epoch = load_epoch();
    // item (i, J): with two buffers, prefetch the next item into the other
    // buffer, then process this one with split J's state; with one, process
    // it, then load the next
    auto item = [&](auto jc, int i) __attribute__((always_inline)) {
      constexpr int J = decltype(jc)::value;
      constexpr int kNj = (J + 1) % SPW;
      PageRegs<FP8>& cur = kOneBuf ? A : pick<J % 2 == 0>(A, B);
      PageRegs<FP8>& nxt = kOneBuf ? A : pick<J % 2 == 0>(B, A);
      VPage& dcur = kOneBuf ? dA : pick<J % 2 == 0>(dA, dB);
      VPage& dnxt = kOneBuf ? dA : pick<kNj % 2 == 0>(dA, dB);
      const int ni = J + 1 < SPW ? i : i + 1;
      if (!kOneBuf && real(kNj, ni)) {
        dnxt = vpage_at(v0s[kNj], k_at(kNj, ni));
        load_vpage<FP8>(nxt, dnxt.r0, dnxt.r1, dnxt.b, lane);
      }
      const bool rl = real(J, i);
      if (patch && rl && i == 0 && J == j_tok) {
        const int id_tok = pt_lds ? uniform_i32(sm_pt[win.pgl]) : pt[win.pgl];
        uint8_t* rec = const_cast<uint8_t*>(head_base) + (int64_t)id_tok * a.page_bytes;
        put_new_token<FP8>(cur, rec, tok, a.rope_cos != nullptr, p, lane, sm_tok[w]);
      }
      process_page<G, FP8>(cur, qr, qh, rl ? dcur.mask : 0u, rl ? dcur.b : 0, a.scale_log2, lane, m_s[J], l_s[J],
                           acc_s[J]);
      if (kOneBuf && real(kNj, ni)) {
        dnxt = vpage_at(v0s[kNj], k_at(kNj, ni));
        load_vpage<FP8>(nxt, dnxt.r0, dnxt.r1, dnxt.b, lane);
      }
    };
    for (int i = 0; i < nw_max; ++i) {
      item(SplitIndex<0>{}, i);
      item(SplitIndex<1>{}, i);
      if constexpr (SPW == 4) {
        item(SplitIndex<2>{}, i);
        item(SplitIndex<3>{}, i);
      }
    }

    asm volatile("" : "+v"(epoch));
    GW_TRACE_T(a, 4, tid == 0);
    GW_TRACE_T(a, 8 + w, lane == 0);
    GW_TRACE_V(a, 1, tid == 0, (uint64_t)nws[0] | (uint64_t)nsplit << 16);
    // ---- per split, merge the waves in LDS, in wave order
    __shared__ float sm_acc_s[SPW][kLocalWaves][G][kLocalD];
    __shared__ float sm_m_s[SPW][kLocalWaves][G], sm_l_s[SPW][kLocalWaves][G];
    __shared__ int sm_last_s;
#pragma unroll
    for (int j = 0; j < SPW; ++j)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float lv = (c == 0) ? l_s[j][h] : 0.f;   // one lane per token slot
        lv += shfl_xor_f32(lv, 4);
        lv += shfl_xor_f32(lv, 8);
        lv += shfl_xor_f32(lv, 16);
        lv += shfl_xor_f32(lv, 32);
        if (lane == 0) {
          sm_m_s[j][w][h] = m_s[j][h];
          sm_l_s[j][w][h] = lv;
        }
        *reinterpret_cast<f32x4*>(&sm_acc_s[j][w][h][4 * lane]) =
            f32x4{acc_s[j][h][0], acc_s[j][h][1], acc_s[j][h][2], acc_s[j][h][3]};
      }
    __syncthreads();
    const bool dt = tid < kLocalD;
    const int d = dt ? tid : 0;
    float o[SPW][G], M[SPW][G], lsum[SPW][G];
#pragma unroll
    for (int j = 0; j < SPW; ++j)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        M[j][h] = sm_m_s[j][0][h];
#pragma unroll
        for (int ww = 1; ww < kLocalWaves; ++ww) M[j][h] = fmaxf(M[j][h], sm_m_s[j][ww][h]);
        lsum[j][h] = 0.f;
        o[j][h] = 0.f;
#pragma unroll
        for (int ww = 0; ww < kLocalWaves; ++ww) {
          const float mw = sm_m_s[j][ww][h];
          const float sw = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M[j][h]);
          lsum[j][h] += sm_l_s[j][ww][h] * sw;
          o[j][h] += sm_acc_s[j][ww][h][d] * sw;
        }
      }
    GW_TRACE_T(a, 5, tid == 0);
    if (nsplit == 1) {
      if (!dt) return;
#pragma unroll
      for (int h = 0; h < G; ++h)
        a.out[((int64_t)row * a.num_q_heads + g * G + h) * kLocalD + d] = o[0][h] / lsum[0][h];
      GW_TRACE_T(a, 7, tid == 0);
      return;
    }
    if (covers_all) {
      // the row's splits merged here, as merge_splits merges published ones
      if (!dt) return;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float Mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < SPW; ++j)
          if (j < nsplit) Mx = fmaxf(Mx, M[j][h]);
        float ls = 0.f, ov = 0.f;
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
          if (j < nsplit) {
            const float sw = __builtin_amdgcn_exp2f(M[j][h] - Mx);
            ls += lsum[j][h] * sw;
            ov += o[j][h] * sw;
          }
        }
        a.out[((int64_t)row * a.num_q_heads + g * G + h) * kLocalD + d] = ov / ls;
      }
      GW_TRACE_T(a, 7, tid == 0);
      return;
    }
    // ---- publish this workgroup's splits; the last workgroup of the
    // (sequence, KV head) to arrive reduces all of them, as with one split
    // per workgroup (the counter counts splits)
    const uint64_t tag = (uint64_t)(epoch + 1u) << 32;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      if (j >= n_own || !dt) break;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const int64_t pi = ((int64_t)s * a.num_q_heads + g * G + h) * a.max_splits + split + j;
        __hip_atomic_store(a.part_acc + pi * kLocalD + d, tag | f32_to_bits(o[j][h]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0) {
          __hip_atomic_store(a.part_ml + pi * 2 + 0, tag | f32_to_bits(M[j][h]), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(a.part_ml + pi * 2 + 1, tag | f32_to_bits(lsum[j][h]), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    lds_barrier();
    int* counter = a.counters + (int64_t)s * a.num_kv_heads + g;
    if (tid == 0)
      sm_last_s = __hip_atomic_fetch_add(counter, n_own, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nsplit - n_own;
    lds_barrier();
    GW_TRACE_T(a, 6, tid == 0);
    if (!sm_last_s || !dt) {
      GW_TRACE_T(a, 7, tid == 0);
      return;
    }
    if (nsplit <= 4) {
      merge_splits<G, 4>(a, s, g * G, row, d, nsplit, tag);
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) merge_splits<1, kLocalMaxSplits>(a, s, g * G + h, row, d, nsplit, tag);
    }
    if (tid == 0) {   // ready for the next call
      __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.epochs + (int64_t)s * a.num_kv_heads + g, epoch + 1u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    GW_TRACE_V(a, 1, tid == 0, (uint64_t)nws[0] | (uint64_t)nsplit << 16 | 1ull << 32);
    GW_TRACE_T(a, 7, tid == 0);
  }
}

}  // namespace

hipError_t launch_local_decode(const LocalAttnArgs& a, int group, bool fp8, hipStream_t stream) {
  const int spw = a.splits_per_wg;
  // the decode items, then the prompt rows' append units (256 threads each)
  const int64_t n_dec = (int64_t)cdiv_i(a.max_splits, spw) * a.num_kv_heads * a.num_seqs;
  const int per_wg = 64 * local_waves(group) / 256;
  const int64_t n = n_dec + (a.append_units + per_wg - 1) / per_wg;
  if (n > 0x7fffffff) return hipErrorInvalidConfiguration;
  LocalAttnArgs b = a;
  b.append_wg0 = (int32_t)n_dec;
  dim3 grid((unsigned)n);
#define GW_LOCAL_CASE(G_, F_, S_)                                                                           \
  if (group == G_ && fp8 == F_ && spw == S_) {                                                              \
    hipLaunchKernelGGL((local_decode_kernel<G_, F_, S_>), grid, dim3(64 * local_waves(G_)), 0, stream, b); \
    return hipGetLastError();                                                                               \
  }
  // the multi-split variants that fit the registers (local_max_splits_per_wg)
  GW_LOCAL_CASE(1, false, 1) GW_LOCAL_CASE(2, false, 1) GW_LOCAL_CASE(4, false, 1)
  GW_LOCAL_CASE(1, true, 1) GW_LOCAL_CASE(2, true, 1) GW_LOCAL_CASE(4, true, 1)
  GW_LOCAL_CASE(4, false, 2)
  GW_LOCAL_CASE(1, true, 2) GW_LOCAL_CASE(2, true, 2) GW_LOCAL_CASE(4, true, 2)
  GW_LOCAL_CASE(4, true, 4)
#undef GW_LOCAL_CASE
  return hipErrorInvalidValue;
}

}  // namespace gw
