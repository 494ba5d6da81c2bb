// KV append (the prep step before attention) and rotary tables.
//
// pegainfer PR #1012, Description: the prep kernel rotates K and stores K/V
// into the pool with the store type (bf16 or e4m3) as a parameter.
// pegainfer "Gemma 4" page, Architecture notes: local K rotates all 256 dims
// (theta 1e4); global K rotates its first 128 of 512 dims (theta 1e6) with
// the frequency denominator kept at 512.  Gewell post, "the Why": global K
// and V are tied, so the global record is V plus the rotated quarter of K.
//
// Rotation pairs (i, i + R/2) inside the rotated block (rotate-half), in
// fp32 from fp32 cos/sin tables; results round to bf16 (nearest even) and,
// for the e4m3 pool, that bf16 value rounds once more to e4m3 (nearest even,
// saturating).  Placement follows the in-page element orders of gw.h.

#include "gw_device.h"
#include "gw_kernels.h"

namespace gw {
namespace {

// ------------------------------------------------------------ rope table --
__global__ void rope_table_kernel(float* cos_out, float* sin_out, int max_pos, int half,
                                  int head_dim, double theta) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)max_pos * half) return;
  const int p = (int)(idx / half), i = (int)(idx % half);
  const double inv = pow(theta, -2.0 * (double)i / (double)head_dim);
  const double ang = (double)p * inv;
  cos_out[idx] = (float)cos(ang);
  sin_out[idx] = (float)sin(ang);
}

__device__ __forceinline__ void load4_bf16(const uint16_t* p, float (&x)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
}

// ------------------------------------------------------ local family -----
// One wave per (token, KV head).  Lane l < 32 rotates pairs i = 4l..4l+3,
// i.e. dims 4l..4l+3 with their partners 128+4l..; every lane stores V
// dims 4l..4l+3.
template <bool FP8, bool ROPE>
__global__ __launch_bounds__(64) void append_local_kernel(AppendArgs a) {
  const int tok = blockIdx.x, h = blockIdx.y, l = threadIdx.x;
  const int s = a.seq_idx[tok], ps = a.pos[tok];
  const int page = a.page_table[(int64_t)s * a.pt_stride + (ps >> 4)];
  const int slot = ps & 15;
  uint8_t* hb = a.pool + (int64_t)page * a.page_bytes + (int64_t)h * a.head_bytes;
  const int64_t src = ((int64_t)tok * a.num_kv_heads + h) * 256;

  if (l < 32) {
    float xa[4], xb[4];
    load4_bf16(a.k_raw + src + 4 * l, xa);
    load4_bf16(a.k_raw + src + 128 + 4 * l, xb);
    float ya[4], yb[4];
    if constexpr (ROPE) {
      const float4 cs = *reinterpret_cast<const float4*>(a.rope_cos + (int64_t)ps * 128 + 4 * l);
      const float4 sn = *reinterpret_cast<const float4*>(a.rope_sin + (int64_t)ps * 128 + 4 * l);
      const float c4[4] = {cs.x, cs.y, cs.z, cs.w}, s4[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) rope_pair(xa[j], xb[j], c4[j], s4[j], ya[j], yb[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) { ya[j] = xa[j]; yb[j] = xb[j]; }
    }
    // dims d = 4l..4l+3 (quarter c = l/16) and d + 128 (quarter c + 2)
    const int c = l >> 4;
    if constexpr (!FP8) {
      const int k = (l & 15) >> 1, e0 = 4 * (l & 1);
      uint16_t* kb = reinterpret_cast<uint16_t*>(hb);
      const uint2 va = {pack_bf16(ya[0], ya[1]), pack_bf16(ya[2], ya[3])};
      const uint2 vb = {pack_bf16(yb[0], yb[1]), pack_bf16(yb[2], yb[3])};
      *reinterpret_cast<uint2*>(kb + ((k * 16 + slot) * 4 + c) * 8 + e0) = va;
      *reinterpret_cast<uint2*>(kb + ((k * 16 + slot) * 4 + c + 2) * 8 + e0) = vb;
    } else {
      const int k = (l & 15) >> 2, e0 = 4 * (l & 3);
      uint32_t wa = 0, wb = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wa |= f32_to_e4m3(round_bf16(ya[j])) << (8 * j);
        wb |= f32_to_e4m3(round_bf16(yb[j])) << (8 * j);
      }
      *reinterpret_cast<uint32_t*>(hb + ((k * 16 + slot) * 4 + c) * 16 + e0) = wa;
      *reinterpret_cast<uint32_t*>(hb + ((k * 16 + slot) * 4 + c + 2) * 16 + e0) = wb;
    }
  }

  // V: dims 4l + j, token slot -> interleaved pairs (bf16) or quads (e4m3)
  float xv[4];
  load4_bf16(a.v + src + 4 * l, xv);
  if constexpr (!FP8) {
    uint16_t* vb = reinterpret_cast<uint16_t*>(hb + 8192);
    const int u = slot >> 1, i = slot & 1;
    const uint2 raw = *reinterpret_cast<const uint2*>(a.v + src + 4 * l);
    const uint16_t e[4] = {(uint16_t)(raw.x & 0xffff), (uint16_t)(raw.x >> 16),
                           (uint16_t)(raw.y & 0xffff), (uint16_t)(raw.y >> 16)};
#pragma unroll
    for (int j = 0; j < 4; ++j) vb[((u * 64 + l) * 4 + j) * 2 + i] = e[j];
    (void)xv;
  } else {
    uint8_t* vb = hb + 4096;
    const int u = slot >> 2, i = slot & 3;
#pragma unroll
    for (int j = 0; j < 4; ++j) vb[((u * 64 + l) * 4 + j) * 4 + i] = (uint8_t)f32_to_e4m3(xv[j]);
  }
}

// ----------------------------------------------------- global family -----
// One wave per token.  Lane l holds V dims 8l..8l+7 (chunk l).  Lanes 0..7
// rotate chunk l with its rotate-half partner chunk l + 8 (pairs (i, i+64),
// i < 64).  COMPRESSED: page = V[16][512] | K_rot[16][128]; FULL: page =
// K[16][512] | V[16][512]; blocks chunk-major ((c*16 + t)*8 + e), or with
// FP8 the e4m3 codes of the same bf16 record in 16-dim chunks.
template <bool COMPRESSED, bool FP8>
__global__ __launch_bounds__(64) void append_global_kernel(AppendArgs a) {
  const int tok = blockIdx.x, l = threadIdx.x;
  const int s = a.seq_idx[tok], ps = a.pos[tok];
  const int page = a.page_table[(int64_t)s * a.pt_stride + (ps >> 4)];
  const uint16_t* vsrc = a.v + (int64_t)tok * 512;
  const uint16_t* ksrc = a.k_raw ? a.k_raw + (int64_t)tok * 512 : vsrc;
  const GlobalRecordLane r = global_record_lane(vsrc, ksrc, a.rope_cos, a.rope_sin, ps, l);
  put_global_record_as<COMPRESSED, FP8>(a.pool + (int64_t)page * a.page_bytes, r, ps & 15, l);
}

}  // namespace

hipError_t launch_rope_table(float* cos_out, float* sin_out, int max_pos, int rot_dim,
                             int head_dim, double theta, hipStream_t stream) {
  const int half = rot_dim / 2;
  const int64_t n = (int64_t)max_pos * half;
  const int block = 256;
  const int64_t grid = (n + block - 1) / block;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)grid), dim3(block), 0, stream, cos_out,
                     sin_out, max_pos, half, head_dim, theta);
  return hipGetLastError();
}

hipError_t launch_append_local(const AppendArgs& a, bool fp8, bool rope, hipStream_t stream) {
  dim3 grid(a.n_tok, a.num_kv_heads), block(64);
  if (fp8) {
    if (rope) hipLaunchKernelGGL((append_local_kernel<true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((append_local_kernel<true, false>), grid, block, 0, stream, a);
  } else {
    if (rope) hipLaunchKernelGGL((append_local_kernel<false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((append_local_kernel<false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_append_global(const AppendArgs& a, bool compressed, bool fp8, hipStream_t stream) {
  dim3 grid(a.n_tok), block(64);
  if (fp8) {
    if (compressed) hipLaunchKernelGGL((append_global_kernel<true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((append_global_kernel<false, true>), grid, block, 0, stream, a);
  } else {
    if (compressed) hipLaunchKernelGGL((append_global_kernel<true, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((append_global_kernel<false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace gw
