// Local-family paged decode attention (sliding window, head dim 256, grouped
// query heads) and the cross-split reduce shared with the global family.
//
// What is computed (pegainfer "Gemma 4" page, intro and Architecture notes;
// pegainfer PR #1012, Description, for the e4m3 pool): for each decode row of
// sequence s at position p = seq_len - 1 and each q head h of KV head
// g = h / G, softmax over the keys j in [max(0, p - W + 1), p] of
// scale * q_h . K_j, applied to V_j, with K/V read from 16-token pages.
//
// Work split: one workgroup per (split, KV head, sequence); a split is a
// balanced run of the pages of the row's window (gw_plan.h).  Four waves per
// workgroup take every fourth page of the split, each with its own online
// softmax state (running max m, sum l, accumulator), merged in LDS at the end.
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

namespace gw {
namespace {

constexpr int kLocalD = 256;
constexpr int kLocalWaves = 4;

template <bool FP8>
struct LocalLayout {
  static constexpr int kBlockBytes = FP8 ? 4096 : 8192;  // one K or V block of a page
  static constexpr int kLoads = FP8 ? 4 : 8;             // 16-byte loads per block per lane
};

template <bool FP8>
struct PageRegs {
  uint4 k[LocalLayout<FP8>::kLoads];
  uint4 v[LocalLayout<FP8>::kLoads];
};

template <bool FP8>
__device__ __forceinline__ void load_page(PageRegs<FP8>& r, const uint8_t* head_base,
                                          int64_t page_bytes, int phys, int lane) {
  const uint8_t* b = head_base + (int64_t)phys * page_bytes + lane * 16;
#pragma unroll
  for (int k = 0; k < LocalLayout<FP8>::kLoads; ++k) r.k[k] = ld16(b + k * 1024);
#pragma unroll
  for (int u = 0; u < LocalLayout<FP8>::kLoads; ++u)
    r.v[u] = ld16(b + LocalLayout<FP8>::kBlockBytes + u * 1024);
}

__device__ __forceinline__ uint32_t u4_get(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ __forceinline__ void u4_and(uint4& v, uint32_t m) {
  v.x &= m; v.y &= m; v.z &= m; v.w &= m;
}

template <int G, bool FP8>
__device__ __forceinline__ void process_page(PageRegs<FP8>& r, const uint32_t (&qr)[G][32],
                                             int lp, int lo, int p, float scale_log2, int lane,
                                             float (&m_run)[G], float (&l_run)[G],
                                             float (&acc)[G][4]) {
  const int t = lane >> 2;
  // ---- scores: lane (t, c) dots its quarter of K_t with q, then quad sum
  float z[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float s0 = 0.f, s1 = 0.f;
    if constexpr (!FP8) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float& s = (k & 1) ? s1 : s0;
#pragma unroll
        for (int m = 0; m < 4; ++m) s = dot2_bf16(u4_get(r.k[k], m), qr[h][4 * k + m], s);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float& s = (k & 1) ? s1 : s0;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t w = u4_get(r.k[k], m);
          s = dot2_bf16(e4m3x2_to_bf16x2<false>(w), qr[h][8 * k + 2 * m], s);
          s = dot2_bf16(e4m3x2_to_bf16x2<true>(w), qr[h][8 * k + 2 * m + 1], s);
        }
      }
    }
    float s = s0 + s1;
    s += dpp_f32<kQuadSwap1>(s);
    s += dpp_f32<kQuadSwap2>(s);
    z[h] = s;
  }
  const int tok = lp * kPage + t;
  const bool valid = tok >= lo && tok <= p;
#pragma unroll
  for (int h = 0; h < G; ++h) z[h] = valid ? z[h] * scale_log2 : -INFINITY;

  // ---- online softmax: page max, rescale on a new maximum (wave-uniform)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = z[h];
    mx = fmaxf(mx, shfl_xor_f32(mx, 4));
    mx = fmaxf(mx, shfl_xor_f32(mx, 8));
    mx = fmaxf(mx, shfl_xor_f32(mx, 16));
    mx = fmaxf(mx, shfl_xor_f32(mx, 32));
    mx = bits_to_f32((uint32_t)uniform_i32((int)f32_to_bits(mx)));
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
    const float nb = shfl_down_f32(pr, 4);                       // token t + 1
    const uint32_t pair = pack_bf16(pr, nb);
    l_run[h] += bf16_lo(pair);
#pragma unroll
    for (int u = 0; u < 8; ++u) P[h][u] = readlane_u32(pair, 8 * u);
  }

  // ---- V of masked tokens at the window's edge pages is zeroed, so that
  // unwritten or stale slots (possibly NaN) contribute exactly 0.
  const int base_tok = lp * kPage;
  if (base_tok < lo || base_tok + kPage - 1 > p) {
    if constexpr (!FP8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t0 = base_tok + 2 * u;
        const uint32_t m = ((t0 >= lo && t0 <= p) ? 0x0000ffffu : 0u) |
                           ((t0 + 1 >= lo && t0 + 1 <= p) ? 0xffff0000u : 0u);
        u4_and(r.v[u], m);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ti = base_tok + 4 * u + i;
          if (ti >= lo && ti <= p) m |= 0xffu << (8 * i);
        }
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

template <int G, bool FP8>
__global__ __launch_bounds__(256, G >= 4 ? 1 : 2) void local_decode_kernel(LocalAttnArgs a) {
  const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;

  int row = s;
  if (a.q_indptr) {
    row = a.q_indptr[s];
    if (a.q_indptr[s + 1] - row != 1) return;   // rows of prompts go elsewhere
  }
  const int L = a.seq_lens[s];
  const int p = L - 1;
  const int lo = max(0, p - a.window + 1);
  const int pg0 = lo >> 4;
  const int npg = (p >> 4) - pg0 + 1;
  const int nsplit = local_nsplit(npg);
  if (split >= nsplit) return;
  const int my0 = pg0 + split_lo(npg, nsplit, split);
  const int my1 = pg0 + split_lo(npg, nsplit, split + 1);

  // q of the group, this lane's quarter of the dims, as bf16 pairs
  const int c = lane & 3;
  uint32_t qr[G][32];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint16_t* qp = a.q + ((int64_t)row * a.num_q_heads + g * G + h) * kLocalD + 64 * c;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint4 v = ld16_cached(qp + 8 * k);
      qr[h][4 * k + 0] = v.x; qr[h][4 * k + 1] = v.y;
      qr[h][4 * k + 2] = v.z; qr[h][4 * k + 3] = v.w;
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

  const int32_t* pt = a.page_table + (int64_t)s * a.pt_stride;
  const uint8_t* head_base = a.pool + (int64_t)g * a.head_bytes;

  // software pipeline: the next page of this wave is in flight while the
  // current one is processed
  PageRegs<FP8> A, B;
  int i = my0 + w;
  if (i < my1) load_page<FP8>(A, head_base, a.page_bytes, uniform_i32(pt[i]), lane);
  while (i < my1) {
    int n = i + kLocalWaves;
    if (n < my1) load_page<FP8>(B, head_base, a.page_bytes, uniform_i32(pt[n]), lane);
    process_page<G, FP8>(A, qr, i, lo, p, a.scale_log2, lane, m_run, l_run, acc);
    i = n;
    if (i >= my1) break;
    n = i + kLocalWaves;
    if (n < my1) load_page<FP8>(A, head_base, a.page_bytes, uniform_i32(pt[n]), lane);
    process_page<G, FP8>(B, qr, i, lo, p, a.scale_log2, lane, m_run, l_run, acc);
    i = n;
  }

  // ---- merge the four waves in LDS, in wave order
  __shared__ float sm_acc[kLocalWaves][G][kLocalD];
  __shared__ float sm_m[kLocalWaves][G], sm_l[kLocalWaves][G];
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

  const int d = tid;   // 256 threads, one output dim each
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = sm_m[0][h];
#pragma unroll
    for (int ww = 1; ww < kLocalWaves; ++ww) M = fmaxf(M, sm_m[ww][h]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int ww = 0; ww < kLocalWaves; ++ww) {
      const float mw = sm_m[ww][h];
      const float sw = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      lsum += sm_l[ww][h] * sw;
      o += sm_acc[ww][h][d] * sw;
    }
    const int qh = g * G + h;
    if (nsplit == 1) {
      a.out[((int64_t)row * a.num_q_heads + qh) * kLocalD + d] = o / lsum;
    } else {
      const int64_t pi = ((int64_t)s * a.num_q_heads + qh) * a.max_splits + split;
      a.part_acc[pi * kLocalD + d] = o;
      if (d == 0) {
        a.part_ml[pi * 2 + 0] = M;
        a.part_ml[pi * 2 + 1] = lsum;
      }
    }
  }
}

// Cross-split reduce, in split order: M = max m_i, l = sum l_i 2^(m_i - M),
// out = sum acc_i 2^(m_i - M) / l.  One workgroup per (sequence, q head),
// four output dims per thread.
__global__ __launch_bounds__(128) void split_reduce_kernel(ReduceArgs a) {
  const int s = blockIdx.x, h = blockIdx.y;
  int row = s;
  if (a.q_indptr) {
    row = a.q_indptr[s];
    if (a.q_indptr[s + 1] - row != 1) return;
  }
  const int L = a.seq_lens[s];
  int nsplit;
  if (a.window > 0) {
    nsplit = local_nsplit(local_range_pages(L - 1, a.window));
  } else {
    nsplit = global_nsplit(cdiv_i(cdiv_i(L, kPage), kGlobalTilePages));
  }
  if (nsplit <= 1) return;
  const int64_t base = ((int64_t)s * a.num_q_heads + h) * a.max_splits;
  float M = -INFINITY;
  for (int i = 0; i < nsplit; ++i) M = fmaxf(M, a.part_ml[(base + i) * 2]);
  float lsum = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  const int d4 = threadIdx.x * 4;
  for (int i = 0; i < nsplit; ++i) {
    const float sw = __builtin_amdgcn_exp2f(a.part_ml[(base + i) * 2] - M);
    lsum += a.part_ml[(base + i) * 2 + 1] * sw;
    const f32x4 v = *reinterpret_cast<const f32x4*>(a.part_acc + (base + i) * a.head_dim + d4);
    o += v * sw;
  }
  *reinterpret_cast<f32x4*>(a.out + ((int64_t)row * a.num_q_heads + h) * a.head_dim + d4) = o / lsum;
}

}  // namespace

hipError_t launch_local_decode(const LocalAttnArgs& a, int group, bool fp8, hipStream_t stream) {
  dim3 grid(a.max_splits, a.num_kv_heads, a.num_seqs), block(256);
#define GW_LOCAL_CASE(G_, F_) \
  if (group == G_ && fp8 == F_) { hipLaunchKernelGGL((local_decode_kernel<G_, F_>), grid, block, 0, stream, a); return hipGetLastError(); }
  GW_LOCAL_CASE(1, false) GW_LOCAL_CASE(2, false) GW_LOCAL_CASE(4, false)
  GW_LOCAL_CASE(1, true) GW_LOCAL_CASE(2, true) GW_LOCAL_CASE(4, true)
#undef GW_LOCAL_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_split_reduce(const ReduceArgs& a, int num_seqs, hipStream_t stream) {
  dim3 grid(num_seqs, a.num_q_heads), block(a.head_dim / 4);
  hipLaunchKernelGGL(split_reduce_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace gw
