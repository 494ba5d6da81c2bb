// Local-family attention of prompt rows (sequences with more than one query
// row in the call): sliding window, head dim 256, grouped query heads, bf16
// or e4m3 pool.
//
// What is computed (pegainfer "Gemma 4" page, Scheduling: a new prompt's rows
// are computed in the same step as the live streams' next token; intro and
// Architecture notes for the window and the grouped heads): row r of
// sequence s sits at position p_r = seq_len - q_len + r; each q head h of
// KV head g = h / G attends the keys j in [max(0, p_r - W + 1), p_r].
//
// With many rows per KV head the score and value steps are dense
// contractions, so both run on MFMA in 16 x 16 blocks over "query vectors"
// (a row and one head of its group): lane column l16 of a wave is query
// vector (row r0 + l16 / G, head l16 % G).
//   S^T (16 tokens x 16 q vectors) = K (16 x 256) . Q^T (256 x 16)
//                                     -- v_mfma_f32_16x16x32_bf16, 8 steps
//   O^T (16 dims x 16 q vectors)  += V^T (16 x 16 tokens) . P^T (16 x 16)
//                                     -- v_mfma_f32_16x16x16_bf16, 16 dim blocks
// A workgroup (4 waves, 64 query vectors) takes 64 / G consecutive rows of
// one (sequence, KV head) and streams the pages of their union range,
// [max(0, p_first - W + 1), p_last], through an LDS ring (direct global->LDS
// transfers, each wave moving a quarter of every page).  Each lane masks its
// own query vector's window; V of tokens outside the union range (slots that
// may never have been written) is zeroed in the operand registers.  e4m3
// codes convert to bf16 exactly (v_cvt_scalef32_pk_bf16_fp8, scale 1), so
// the products are the same as on the bf16 values.  P is rounded to bf16 for
// PV and the sum l adds exactly those rounded values.  The row blocks with
// the longest ranges are dispatched first.

#include "gw_device.h"
#include "gw_kernels.h"
#include "gw_plan.h"

namespace gw {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <bool FP8>
struct LocalHead {
  static constexpr int kBytes = FP8 ? 8192 : 16384;   // K block + V block of one KV head
  static constexpr int kVOff = kBytes / 2;
  // K operand: token t, dims 32 ks + 8 gq .. +7, as 8 bf16
  __device__ static __forceinline__ bf16x8 k_frag(const uint8_t* pg, int ks, int gq, int t) {
    if constexpr (!FP8) {
      const int k = 4 * (ks & 1) + gq, c = ks >> 1;
      return *reinterpret_cast<const bf16x8*>(pg + ((k * 16 + t) * 4 + c) * 16);
    } else {
      const int k = 2 * (ks & 1) + (gq >> 1), c = ks >> 1;
      const uint2 w = *reinterpret_cast<const uint2*>(pg + ((k * 16 + t) * 4 + c) * 16 + 8 * (gq & 1));
      return __builtin_bit_cast(bf16x8, uint4{e4m3x2_to_bf16x2<false>(w.x), e4m3x2_to_bf16x2<true>(w.x),
                                              e4m3x2_to_bf16x2<false>(w.y), e4m3x2_to_bf16x2<true>(w.y)});
    }
  }
  // V^T operand: dim d, tokens 4 gq .. 4 gq + 3, as 4 bf16 (two dwords)
  __device__ static __forceinline__ uint2 v_frag(const uint8_t* pg, int d, int gq) {
    if constexpr (!FP8) {
      const uint8_t* b = pg + kVOff + (((2 * gq) * 64 + (d >> 2)) * 4 + (d & 3)) * 4;
      return uint2{*reinterpret_cast<const uint32_t*>(b), *reinterpret_cast<const uint32_t*>(b + 1024)};
    } else {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(pg + kVOff + ((gq * 64 + (d >> 2)) * 4 + (d & 3)) * 4);
      return uint2{e4m3x2_to_bf16x2<false>(w), e4m3x2_to_bf16x2<true>(w)};
    }
  }
};

template <int G, bool FP8, int NS>
__global__ __launch_bounds__(256, 2) void local_prefill_kernel(LocalAttnArgs a) {
  using LH = LocalHead<FP8>;
  constexpr int kUnits = LH::kBytes / 1024;   // 1 KiB transfer units per (page, head)
  constexpr int kPerWave = kUnits / 4;
  constexpr int kRowsPerWave = 16 / G;
  constexpr int kRowsPerWG = 4 * kRowsPerWave;
  static_assert(NS >= 2 && NS - 2 <= 4 && kPerWave * (NS - 2) < 64, "ring depth");
  __shared__ __attribute__((aligned(16))) uint8_t ring[NS][LH::kBytes];

  const int s = blockIdx.x, gk = blockIdx.y;
  const int row0 = a.q_indptr[s];
  const int q_len = a.q_indptr[s + 1] - row0;
  if (q_len < 2) return;
  const int rb = cdiv_i(q_len, kRowsPerWG) - 1 - (int)blockIdx.z;   // longest ranges first
  if (rb < 0) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = uniform_i32(tid >> 6);
  const int gq = lane >> 4, l16 = lane & 15;
  const int L = a.seq_lens[s];
  const int r_first = rb * kRowsPerWG;
  const int r_last = min(r_first + kRowsPerWG, q_len) - 1;
  const int p_last = L - q_len + r_last;
  const int lo_first = max(0, L - q_len + r_first - a.window + 1);
  const int pg_lo = lo_first >> 4;
  const int n = (p_last >> 4) - pg_lo + 1;

  // this lane's query vector
  const int r = r_first + w * kRowsPerWave + l16 / G, hq = l16 % G;
  const bool row_ok = r <= r_last;
  const int rr = row_ok ? r : r_last;
  const int pq = L - q_len + rr;
  const int loq = max(0, pq - a.window + 1);

  PageIds ids;
  ids.init(a.page_table + (int64_t)s * a.pt_stride + pg_lo, n, lane);
  const uint32_t ring_base = uniform_i32((int)lds_address(&ring[0][0])) + (uint32_t)(1024 * kPerWave * w);
  const int64_t head_off = (int64_t)gk * a.head_bytes + 1024 * kPerWave * w + 16 * lane;
  auto issue_page = [&](int i) __attribute__((always_inline)) {
    const uint8_t* src = a.pool + (int64_t)ids.get(i) * a.page_bytes + head_off;
    const uint32_t dst = ring_base + (uint32_t)((i % NS) * LH::kBytes);
#pragma unroll
    for (int u = 0; u < kPerWave; ++u) dma16_to_lds(src + 1024 * u, dst + 1024 * u);
  };
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (i < n) issue_page(i);

  // Q^T operand: query vector l16, dims 32 ks + 8 gq .. +7
  bf16x8 qf[8];
  {
    const uint16_t* qp = a.q + ((int64_t)(row0 + rr) * a.num_q_heads + gk * G + hq) * 256 + 8 * gq;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ld16_cached(qp + 32 * ks));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  f32x4 acc[16];
#pragma unroll
  for (int b = 0; b < 16; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int i = 0; i < n; ++i) {
    wait_groups_after<kPerWave>(min(NS - 2, n - 1 - i));
    lds_barrier();   // page i is in LDS for every wave; page i - 1 is done
    if (i + NS - 1 < n) issue_page(i + NS - 1);
    const uint8_t* pg = ring[i % NS];
    const int tok_page0 = (pg_lo + i) * 16;

    // ---- S^T = K . Q^T (two accumulation chains)
    bf16x8 kf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kf[ks] = LH::k_frag(pg, ks, gq, l16);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int ks = 0; ks < 8; ks += 2) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks + 1], qf[ks + 1], s1, 0, 0, 0);
    }
    const f32x4 sacc = s0 + s1;

    // ---- online softmax of this lane's query vector over the page
    const int tok0 = tok_page0 + 4 * gq;
    float z[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      z[k] = (row_ok && tok0 + k >= loq && tok0 + k <= pq) ? sacc[k] * a.scale_log2 : -INFINITY;
    const float mx = max_lanes_xor16_32(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
    const float mnew = fmaxf(m_run, mx);
    if (__any(mnew > m_run)) {
      const float alpha = mnew > m_run ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.f;
#pragma unroll
      for (int b = 0; b < 16; ++b) acc[b] *= alpha;
      l_run *= alpha;
    }
    m_run = mnew;
    float pr[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) pr[k] = z[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[k] - m_run);
    const uint32_t p01 = pack_bf16(pr[0], pr[1]), p23 = pack_bf16(pr[2], pr[3]);
    l_run += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
    const s16x4 pb = __builtin_bit_cast(s16x4, uint2{p01, p23});

    // ---- O^T += V^T . P^T; V of tokens outside the union range is zeroed
    uint32_t vm0 = 0xffffffffu, vm1 = 0xffffffffu;
    if (tok_page0 < lo_first || tok_page0 + 15 > p_last) {
      auto in = [&](int t) { return t >= lo_first && t <= p_last; };
      vm0 = (in(tok0) ? 0x0000ffffu : 0u) | (in(tok0 + 1) ? 0xffff0000u : 0u);
      vm1 = (in(tok0 + 2) ? 0x0000ffffu : 0u) | (in(tok0 + 3) ? 0xffff0000u : 0u);
    }
    uint2 vf[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) vf[b] = LH::v_frag(pg, 16 * b + l16, gq);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      uint2 vv = vf[b];
      vv.x &= vm0;
      vv.y &= vm1;
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vv), pb, acc[b], 0, 0, 0);
    }
  }

  // ---- write: lane holds query vector l16, dims 16 b + 4 gq .. +3
  const float l_tot = sum_lanes_xor16_32(l_run);
  if (!row_ok) return;
  float* op = a.out + ((int64_t)(row0 + r) * a.num_q_heads + gk * G + hq) * 256 + 4 * gq;
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int b = 0; b < 16; ++b) *reinterpret_cast<f32x4*>(op + 16 * b) = acc[b] * inv;
}

}  // namespace

hipError_t launch_local_prefill(const LocalAttnArgs& a, int group, bool fp8, int max_q_len,
                                hipStream_t stream) {
  const int rows_per_wg = 64 / group;
  dim3 grid(a.num_seqs, a.num_kv_heads, (max_q_len + rows_per_wg - 1) / rows_per_wg), block(256);
#define GW_PREFILL_CASE(G_, F_) \
  if (group == G_ && fp8 == F_) { hipLaunchKernelGGL((local_prefill_kernel<G_, F_, 4>), grid, block, 0, stream, a); return hipGetLastError(); }
  GW_PREFILL_CASE(1, false) GW_PREFILL_CASE(2, false) GW_PREFILL_CASE(4, false)
  GW_PREFILL_CASE(1, true) GW_PREFILL_CASE(2, true) GW_PREFILL_CASE(4, true)
#undef GW_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace gw
