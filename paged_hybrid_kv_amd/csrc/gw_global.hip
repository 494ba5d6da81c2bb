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
// contractions (32 heads x 16 tokens x 512 dims per page), so both run on
// MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//   S^T (32 tokens x 32 heads) = K (32 x 512) . Q^T (512 x 32)
//   O^T (512 dims x 32 heads) += V^T (512 x 32 tokens) . P^T (32 x 32 heads)
// Work split: one workgroup per (split, sequence); a split is a balanced run
// of 2-page tiles (gw_plan.h).  The four waves of a workgroup each own 128
// of the 512 dims: wave w forms the partial S over its dims (wave 0 from the
// K_rot block, waves 1-3 from V, read once for both products), the partials
// are summed in LDS in wave order, and every wave then runs the same online
// softmax and accumulates its 128 output dims.  V reaches the PV operand
// layout (8 consecutive tokens of one dim per lane) through a wave-private
// LDS transpose.
//
// Lane roles: with l32 = lane % 32 and hf = lane / 32, the S output gives
// lane (l32, hf) head l32 and tokens 8(r/4) + 4hf + r%4 (r < 16); those same
// registers, rounded to bf16 pairs, are the P operand of the PV product, by
// ordering its 16-token contraction as slot (8hf + e) of step ks <-> token
// 16ks + 8(e/4) + 4hf + e%4.  P's rounding is also what the sum l adds.

#include "gw_device.h"
#include "gw_kernels.h"
#include "gw_plan.h"

namespace gw {
namespace {

constexpr int kGD = 512;
constexpr int kGWaves = 4;
constexpr int kVtStride = 40;    // uint16 per row of the V^T tile (32 used; 80-byte rows)

// token <-> PV contraction slot: swap bits 2 and 3
__device__ __forceinline__ int slot_of_token(int t) {
  return (t & ~0xC) | ((t & 4) << 1) | ((t & 8) >> 1);
}

struct TileRegs {
  uint4 k[8];
  uint4 v[8];
};

// Write a wave's V fragments (token l32, dims 16kc + 8hf + e) transposed into
// its LDS tile: row = local dim, column = contraction slot of the token.
__device__ __forceinline__ void stage_vt(uint16_t (*vt)[kVtStride], const uint4 (&src)[8], bool zero,
                                         int hf, int l32) {
  const int col = slot_of_token(l32);
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    uint32_t d4[4] = {src[kc].x, src[kc].y, src[kc].z, src[kc].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) d4[j] = zero ? 0u : d4[j];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t wv = d4[e >> 1];
      vt[16 * kc + 8 * hf + e][col] = (uint16_t)((e & 1) ? (wv >> 16) : (wv & 0xffff));
    }
  }
}

template <bool COMPRESSED>
__global__ __launch_bounds__(256, 1) void global_decode_kernel(GlobalAttnArgs a) {
  const int split = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int hf = lane >> 5, l32 = lane & 31;

  int row = s;
  if (a.q_indptr) {
    row = a.q_indptr[s];
    if (a.q_indptr[s + 1] - row != 1) return;
  }
  const int L = a.seq_lens[s];
  const int p = L - 1;
  const int n_pages = (p >> 4) + 1;
  const int n_tiles = cdiv_i(n_pages, kGlobalTilePages);
  const int nsplit = global_nsplit(n_tiles);
  if (split >= nsplit) return;
  const int t0 = split_lo(n_tiles, nsplit, split);
  const int t1 = split_lo(n_tiles, nsplit, split + 1);

  __shared__ __attribute__((aligned(16))) float sbuf[2][kGWaves][64][16];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kGWaves][128][kVtStride];

  // ---- Q fragments (B operand of S^T): head l32, dims 128w + 16kc + 8hf + e
  bf16x8 qf[8];
  {
    const bool head_ok = l32 < a.num_q_heads;
    const uint16_t* qp = a.q + ((int64_t)row * a.num_q_heads + (head_ok ? l32 : 0)) * kGD + 128 * w + 8 * hf;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      uint4 v = ld16_cached(qp + 16 * kc);
      if (!head_ok) v = uint4{0u, 0u, 0u, 0u};
      qf[kc] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- where this lane's 16-byte pieces sit inside a page (kc = 0; +512 B per kc)
  const int slot = l32 & 15;
  const int chunk0 = 16 * w + hf;                  // 8-dim chunk of dims 128w + 8hf
  int k_off, v_off;
  if constexpr (COMPRESSED) {
    k_off = (w == 0) ? 16 * 512 * 2 + ((hf * 16) + slot) * 16 : (chunk0 * 16 + slot) * 16;
    v_off = (chunk0 * 16 + slot) * 16;
  } else {
    k_off = (chunk0 * 16 + slot) * 16;
    v_off = 16 * 512 * 2 + k_off;
  }
  const bool sep_v = !COMPRESSED || w == 0;       // V needs its own registers
  const int32_t* pt = a.page_table + (int64_t)s * a.pt_stride;

  auto load_tile = [&](TileRegs& r, int tile) {
    const int lp0 = tile * 2;
    const int ph0 = uniform_i32(pt[lp0]);
    const int ph1 = (lp0 + 1 < n_pages) ? uniform_i32(pt[lp0 + 1]) : ph0;
    const uint8_t* base = a.pool + (int64_t)((l32 < 16) ? ph0 : ph1) * a.page_bytes;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) r.k[kc] = ld16(base + k_off + 512 * kc);
    if (sep_v) {
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) r.v[kc] = ld16(base + v_off + 512 * kc);
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x16{};
  int cur = 0;

  auto process_tile = [&](TileRegs& r, int tile) {
    // S^T partial over this wave's 128 dims
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int kc = 0; kc < 8; ++kc)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, r.k[kc]), qf[kc], sacc, 0, 0, 0);

    // V of tokens past p (unwritten slots, or the stand-in second page) -> 0,
    // then V^T into this wave's LDS tile (row = local dim, column = slot)
    const int tok0 = tile * 32;
    const bool zero_v = tok0 + l32 > p;
    if (sep_v) stage_vt(vt[w], r.v, zero_v, hf, l32);
    else stage_vt(vt[w], r.k, zero_v, hf, l32);
    // exchange score partials; every wave sums them in wave order
    *reinterpret_cast<f32x4*>(&sbuf[cur][w][lane][0]) = f32x4{sacc[0], sacc[1], sacc[2], sacc[3]};
    *reinterpret_cast<f32x4*>(&sbuf[cur][w][lane][4]) = f32x4{sacc[4], sacc[5], sacc[6], sacc[7]};
    *reinterpret_cast<f32x4*>(&sbuf[cur][w][lane][8]) = f32x4{sacc[8], sacc[9], sacc[10], sacc[11]};
    *reinterpret_cast<f32x4*>(&sbuf[cur][w][lane][12]) = f32x4{sacc[12], sacc[13], sacc[14], sacc[15]};
    __syncthreads();
    float z[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4 v = *reinterpret_cast<const f32x4*>(&sbuf[cur][0][lane][4 * q4]);
#pragma unroll
      for (int ww = 1; ww < kGWaves; ++ww) v += *reinterpret_cast<const f32x4*>(&sbuf[cur][ww][lane][4 * q4]);
#pragma unroll
      for (int j = 0; j < 4; ++j) z[4 * q4 + j] = v[j];
    }
    cur ^= 1;

    // online softmax for head l32 over this lane's 16 tokens (+ partner half)
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tok = tok0 + 8 * (r >> 2) + 4 * hf + (r & 3);
      z[r] = (tok <= p) ? z[r] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, z[r]);
    }
    mx = fmaxf(mx, shfl_xor_f32(mx, 32));
    const float mnew = fmaxf(m_run, mx);
    if (__any(mnew > m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] *= alpha;
      l_run *= alpha;
    }
    m_run = mnew;
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(z[2 * i] - m_run);
      const float p1 = __builtin_amdgcn_exp2f(z[2 * i + 1] - m_run);
      pk[i] = pack_bf16(p0, p1);
      l_run += bf16_lo(pk[i]);
      l_run += bf16_hi(pk[i]);
    }

    // O^T += V^T . P^T over the two 16-token contraction steps
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, uint4{pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]});
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const uint4 av = *reinterpret_cast<const uint4*>(&vt[w][32 * mb + l32][16 * ks + 8 * hf]);
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb, acc[mb], 0, 0, 0);
      }
    }
  };

  TileRegs A, B;
  int tile = t0;
  if (tile < t1) load_tile(A, tile);
  while (tile < t1) {
    int n = tile + 1;
    if (n < t1) load_tile(B, n);
    process_tile(A, tile);
    tile = n;
    if (tile >= t1) break;
    n = tile + 1;
    if (n < t1) load_tile(A, n);
    process_tile(B, tile);
    tile = n;
  }

  // ---- write: lane holds head l32, dims 128w + 32mb + 8g + 4hf + j
  const float l_tot = l_run + shfl_xor_f32(l_run, 32);
  if (l32 >= a.num_q_heads) return;
  if (nsplit == 1) {
    float* op = a.out + ((int64_t)row * a.num_q_heads + l32) * kGD + 128 * w + 4 * hf;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(op + 32 * mb + 8 * g) =
            f32x4{acc[mb][4 * g] / l_tot, acc[mb][4 * g + 1] / l_tot, acc[mb][4 * g + 2] / l_tot,
                  acc[mb][4 * g + 3] / l_tot};
  } else {
    const int64_t pi = ((int64_t)s * a.num_q_heads + l32) * a.max_splits + split;
    float* op = a.part_acc + pi * kGD + 128 * w + 4 * hf;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(op + 32 * mb + 8 * g) =
            f32x4{acc[mb][4 * g], acc[mb][4 * g + 1], acc[mb][4 * g + 2], acc[mb][4 * g + 3]};
    if (w == 0 && hf == 0) {
      a.part_ml[pi * 2 + 0] = m_run;
      a.part_ml[pi * 2 + 1] = l_tot;
    }
  }
}

}  // namespace

hipError_t launch_global_decode(const GlobalAttnArgs& a, bool compressed, hipStream_t stream) {
  dim3 grid(a.max_splits, a.num_seqs), block(256);
  if (compressed) hipLaunchKernelGGL((global_decode_kernel<true>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((global_decode_kernel<false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace gw
