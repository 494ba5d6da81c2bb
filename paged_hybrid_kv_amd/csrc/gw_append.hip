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

// Sequence and position of appended token tok (see AppendArgs); false if
// the token is left to another kernel.  Uniform over the workgroup.
__device__ __forceinline__ bool append_target(const AppendArgs& a, int tok, int& s, int& ps) {
  if (!a.seq_lens) {
    s = a.seq_idx[tok];
    ps = a.pos[tok];
    return true;
  }
  if (!a.q_indptr) {                    // one row per sequence: its last token
    s = tok;
    ps = a.seq_lens[tok] - 1;
    return !a.skip_single;
  }
  int lo = 0, hi = a.num_seqs;          // largest s with q_indptr[s] <= tok
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.q_indptr[mid] <= tok) lo = mid;
    else hi = mid;
  }
  s = lo;
  const int ql = a.q_indptr[s + 1] - a.q_indptr[s];
  if (a.skip_single && ql == 1) return false;
  ps = a.seq_lens[s] - ql + (tok - a.q_indptr[s]);
  return true;
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
  int s, ps;
  if (!append_target(a, tok, s, ps)) return;
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
  int s, ps;
  if (!append_target(a, tok, s, ps)) return;
  const int page = a.page_table[(int64_t)s * a.pt_stride + (ps >> 4)];
  const uint16_t* vsrc = a.v + (int64_t)tok * 512;
  const uint16_t* ksrc = a.k_raw ? a.k_raw + (int64_t)tok * 512 : vsrc;
  const GlobalRecordLane r = global_record_lane(vsrc, ksrc, a.rope_cos, a.rope_sin, ps, l);
  put_global_record_as<COMPRESSED, FP8>(a.pool + (int64_t)page * a.page_bytes, r, ps & 15, l);
}

// ------------------------------------------------ rows of an attention call
// One workgroup per (sequence, page of its rows' range[, KV head]), the
// (sequence, page) pairs numbered compactly: the rows' own tokens that fall
// in that page are rotated and stored with whole 16-byte units where the
// unit's tokens are all rows (everywhere but at the ends of a range), so a
// page of prompt rows is written with coalesced stores, and the page lookup
// is made once per page.  Row r of sequence s is at position
// seq_lens[s] - q_len + r (the attention calls' rows); one-row sequences
// are skipped when skip_single is set (their decode kernel appends them).
// The arithmetic is the per-token kernels' exactly.
struct RowsPage {
  int r0, p0, pg, t0, t1, page;   // first row and its position, page index, slots [t0, t1], physical page
};

// Work item `item` of a rows call: the call's (sequence, page of its rows'
// range) pairs, numbered sequence by sequence (wave 0's lanes scan 64
// sequences at a time).  False when item is past the last pair.
__device__ __forceinline__ bool rows_page(const AppendArgs& a, int item, RowsPage& rp) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int c = 0; c < a.num_seqs; c += 64) {
    const int sl = c + lane;
    int cnt = 0, r0 = 0, ql = 0, L = 0;
    if (sl < a.num_seqs) {
      r0 = a.q_indptr ? a.q_indptr[sl] : sl;
      ql = a.q_indptr ? a.q_indptr[sl + 1] - r0 : 1;
      L = a.seq_lens[sl];
      if (ql > 0 && !(a.skip_single && ql == 1)) cnt = ((L - 1) >> 4) - ((L - ql) >> 4) + 1;
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
      const int s = c + ls;
      const int j = item - (base + __builtin_amdgcn_readlane(incl, ls) - __builtin_amdgcn_readlane(cnt, ls));
      rp.r0 = __builtin_amdgcn_readlane(r0, ls);
      const int Ls = __builtin_amdgcn_readlane(L, ls);
      rp.p0 = Ls - __builtin_amdgcn_readlane(ql, ls);
      rp.pg = (rp.p0 >> 4) + j;
      rp.t0 = max(rp.p0 - rp.pg * kPage, 0);
      rp.t1 = min(Ls - 1 - rp.pg * kPage, kPage - 1);
      rp.page = a.page_table[(int64_t)s * a.pt_stride + rp.pg];
      return true;
    }
    base += total;
  }
  return false;
}

template <int N>
__device__ __forceinline__ void load_bf16_n(const uint16_t* p, float (&x)[N]) {
#pragma unroll
  for (int q = 0; q < N / 8; ++q) {
    const uint4 v = *reinterpret_cast<const uint4*>(p + 8 * q);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      x[8 * q + 2 * m] = bf16_lo(w[m]);
      x[8 * q + 2 * m + 1] = bf16_hi(w[m]);
    }
  }
}

// Local family.  K unit (k, t, c) (16 bytes at ((k*16 + t)*4 + c)*16 of the
// K block) holds dims 64c + W k .. + W-1 of slot t (W = 8 bf16 / 16 e4m3);
// quarters c and c + 2 are rotation partners, so thread (t, k, c < 2)
// makes both.  V unit (u, l) (16 bytes at (u*64 + l)*16 of the V block)
// holds dims 4l .. 4l+3 of slots T u .. T u + T-1 (T = 2 bf16 / 4 e4m3).
// A workgroup takes kRowsHeads KV heads of its page: every head's inputs
// are loaded first, in one round trip, and the rotary factors of a slot
// (the same for every head) once.
constexpr int kRowsHeads = 2;

template <bool FP8, bool ROPE>
__global__ __launch_bounds__(256) void append_local_rows_kernel(AppendArgs a) {
  constexpr int kW = FP8 ? 16 : 8;           // dims per K unit
  constexpr int kU = FP8 ? 4 : 8;            // K units per quarter
  constexpr int kT = FP8 ? 4 : 2;            // slots per V unit
  constexpr int kVOff = FP8 ? 4096 : 8192;
  constexpr int kVUnits = (kPage / kT) * 64;          // V units per (page, head)
  constexpr int kVPer = (kVUnits + 255) / 256;        // V units per thread
  const int h0 = blockIdx.y * kRowsHeads, tid = threadIdx.x;
  RowsPage rp;
  if (!rows_page(a, blockIdx.x, rp)) return;
  auto row_src = [&](int t, int h) __attribute__((always_inline)) {   // element offset of slot t's K / V
    return ((int64_t)(rp.r0 + rp.pg * kPage + t - rp.p0) * a.num_kv_heads + h) * 256;
  };
  // K role of this thread: slot t, unit k, quarter pair c
  const int t = tid / (kU * 2), k = (tid >> 1) % kU, c = tid & 1;
  const bool k_on = tid < kPage * kU * 2 && t >= rp.t0 && t <= rp.t1;
  const int d = 64 * c + kW * k;
  float cs[kW], sn[kW];
  if (ROPE && k_on) {
    const float* cp = a.rope_cos + (int64_t)(rp.pg * kPage + t) * 128 + d;
    const float* sp = a.rope_sin + (int64_t)(rp.pg * kPage + t) * 128 + d;
#pragma unroll
    for (int e = 0; e < kW; e += 4) {
      const float4 c4 = *reinterpret_cast<const float4*>(cp + e);
      const float4 s4 = *reinterpret_cast<const float4*>(sp + e);
      cs[e] = c4.x; cs[e + 1] = c4.y; cs[e + 2] = c4.z; cs[e + 3] = c4.w;
      sn[e] = s4.x; sn[e + 1] = s4.y; sn[e + 2] = s4.z; sn[e + 3] = s4.w;
    }
  }
  // ---- every head's raw inputs
  uint4 kra[kRowsHeads][kW / 8], krb[kRowsHeads][kW / 8];
  uint2 vr[kRowsHeads][kVPer][kT];
#pragma unroll
  for (int i = 0; i < kRowsHeads; ++i) {
    const int h = h0 + i;
    if (h >= a.num_kv_heads) break;
    if (k_on) {
      const uint16_t* kp = a.k_raw + row_src(t, h) + d;
#pragma unroll
      for (int q = 0; q < kW / 8; ++q) {
        kra[i][q] = *reinterpret_cast<const uint4*>(kp + 8 * q);
        krb[i][q] = *reinterpret_cast<const uint4*>(kp + 128 + 8 * q);
      }
    }
#pragma unroll
    for (int j = 0; j < kVPer; ++j) {
      const int un = tid + 256 * j, u = un >> 6, l = un & 63;
#pragma unroll
      for (int e = 0; e < kT; ++e) {
        const int ts = kT * u + e;
        const bool in = un < kVUnits && ts >= rp.t0 && ts <= rp.t1;
        vr[i][j][e] = in ? *reinterpret_cast<const uint2*>(a.v + row_src(ts, h) + 4 * l) : uint2{0u, 0u};
      }
    }
  }
  // ---- rotate, round and store, head by head
#pragma unroll
  for (int i = 0; i < kRowsHeads; ++i) {
    const int h = h0 + i;
    if (h >= a.num_kv_heads) break;
    uint8_t* hb = a.pool + (int64_t)rp.page * a.page_bytes + (int64_t)h * a.head_bytes;
    if (k_on) {
      float xa[kW], xb[kW], ya[kW], yb[kW];
#pragma unroll
      for (int q = 0; q < kW / 8; ++q) {
        const uint32_t wa[4] = {kra[i][q].x, kra[i][q].y, kra[i][q].z, kra[i][q].w};
        const uint32_t wb[4] = {krb[i][q].x, krb[i][q].y, krb[i][q].z, krb[i][q].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          xa[8 * q + 2 * m] = bf16_lo(wa[m]);
          xa[8 * q + 2 * m + 1] = bf16_hi(wa[m]);
          xb[8 * q + 2 * m] = bf16_lo(wb[m]);
          xb[8 * q + 2 * m + 1] = bf16_hi(wb[m]);
        }
      }
      if constexpr (ROPE) {
#pragma unroll
        for (int e = 0; e < kW; ++e) rope_pair(xa[e], xb[e], cs[e], sn[e], ya[e], yb[e]);
      } else {
#pragma unroll
        for (int e = 0; e < kW; ++e) { ya[e] = xa[e]; yb[e] = xb[e]; }
      }
      uint4 ua, ub;
      if constexpr (!FP8) {
        ua = uint4{pack_bf16(ya[0], ya[1]), pack_bf16(ya[2], ya[3]), pack_bf16(ya[4], ya[5]), pack_bf16(ya[6], ya[7])};
        ub = uint4{pack_bf16(yb[0], yb[1]), pack_bf16(yb[2], yb[3]), pack_bf16(yb[4], yb[5]), pack_bf16(yb[6], yb[7])};
      } else {
        uint32_t wa[4], wb[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          wa[q] = wb[q] = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            wa[q] |= f32_to_e4m3(round_bf16(ya[4 * q + e])) << (8 * e);
            wb[q] |= f32_to_e4m3(round_bf16(yb[4 * q + e])) << (8 * e);
          }
        }
        ua = uint4{wa[0], wa[1], wa[2], wa[3]};
        ub = uint4{wb[0], wb[1], wb[2], wb[3]};
      }
      *reinterpret_cast<uint4*>(hb + ((k * kPage + t) * 4 + c) * 16) = ua;
      *reinterpret_cast<uint4*>(hb + ((k * kPage + t) * 4 + c + 2) * 16) = ub;
    }
    // V: kPage / kT x 64 units
#pragma unroll
    for (int j = 0; j < kVPer; ++j) {
      const int un = tid + 256 * j;
      if (un >= kVUnits) continue;
      const int u = un >> 6;
      const int ta = kT * u;
      if (ta + kT - 1 < rp.t0 || ta > rp.t1) continue;
      uint32_t ev[kT][4];   // element jj of slot ta + e, as raw bits (bf16) / e4m3 code
#pragma unroll
      for (int e = 0; e < kT; ++e) {
        const uint2 raw = vr[i][j][e];
        const uint32_t b16[4] = {raw.x & 0xffffu, raw.x >> 16, raw.y & 0xffffu, raw.y >> 16};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) ev[e][jj] = FP8 ? f32_to_e4m3(bits_to_f32(b16[jj] << 16)) : b16[jj];
      }
      uint8_t* ub = hb + kVOff + un * 16;
      if (ta >= rp.t0 && ta + kT - 1 <= rp.t1) {   // the whole unit is rows of this call
        uint32_t wv[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          if constexpr (!FP8) wv[jj] = ev[0][jj] | (ev[1][jj] << 16);
          else wv[jj] = ev[0][jj] | (ev[1][jj] << 8) | (ev[2][jj] << 16) | (ev[3][jj] << 24);
        }
        *reinterpret_cast<uint4*>(ub) = uint4{wv[0], wv[1], wv[2], wv[3]};
      } else {                                     // an end of the range: element by element
#pragma unroll
        for (int e = 0; e < kT; ++e) {
          const int ts = ta + e;
          if (ts < rp.t0 || ts > rp.t1) continue;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            if constexpr (!FP8) reinterpret_cast<uint16_t*>(ub)[jj * 2 + e] = (uint16_t)ev[e][jj];
            else ub[jj * 4 + e] = (uint8_t)ev[e][jj];
          }
        }
      }
    }
  }
}

// Global family.  V unit (c, t) (16 bytes at (c*16 + t)*16 of the V block)
// holds dims 8c .. 8c+7 of slot t; K_rot units (c, t) and (c + 8, t), c < 8,
// hold the rotation of V's chunks c and c + 8 (pairs (i, i + 64)); the full
// record's K block repeats V's chunks 16 .. 63.
template <bool COMPRESSED>
__global__ __launch_bounds__(256) void append_global_rows_kernel(AppendArgs a) {
  const int tid = threadIdx.x;
  RowsPage rp;
  if (!rows_page(a, blockIdx.x, rp)) return;
  uint8_t* pb = a.pool + (int64_t)rp.page * a.page_bytes;
  uint8_t* vblock = COMPRESSED ? pb : pb + 16384;
  uint8_t* kblock = COMPRESSED ? pb + 16384 : pb;
  auto row_v = [&](int t) __attribute__((always_inline)) {
    return a.v + (int64_t)(rp.r0 + rp.pg * kPage + t - rp.p0) * 512;
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int un = tid + 256 * i, c = un >> 4, t = un & 15;
    if (t < rp.t0 || t > rp.t1) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(row_v(t) + 8 * c);
    *reinterpret_cast<uint4*>(vblock + un * 16) = v;
    if (!COMPRESSED && c >= 16) *reinterpret_cast<uint4*>(kblock + un * 16) = v;
  }
  if (tid < 128) {
    const int c = tid >> 4, t = tid & 15;
    if (t >= rp.t0 && t <= rp.t1) {
      const uint16_t* vr = row_v(t);
      const uint16_t* kr = a.k_raw ? a.k_raw + (vr - a.v) : vr;   // the same row of k_raw
      const GlobalRecordLane r = global_record_lane(vr, kr, a.rope_cos, a.rope_sin, rp.pg * kPage + t, c);
      *reinterpret_cast<uint4*>(kblock + (c * 16 + t) * 16) = r.ka;
      *reinterpret_cast<uint4*>(kblock + ((c + 8) * 16 + t) * 16) = r.kb;
    }
  }
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

// Items of a rows call: a sequence of q rows touches at most
// (q + 14) / 16 + 1 pages, so the call at most (rows + 30 sequences) / 16
// (and at most sequences * pages of max_q_len).
static int64_t rows_items(const AppendArgs& a, int max_q_len) {
  const int64_t by_rows = ((int64_t)a.n_tok + 30LL * a.num_seqs) / kPage;
  const int64_t by_len = (int64_t)a.num_seqs * ((max_q_len + 14) / kPage + 1);
  return by_rows < by_len ? by_rows : by_len;
}

hipError_t launch_append_local_rows(const AppendArgs& a, bool fp8, bool rope, int max_q_len, hipStream_t stream) {
  const int64_t items = rows_items(a, max_q_len);
  if (items == 0) return hipSuccess;
  if (items > 0x7fffffff) return launch_append_local(a, fp8, rope, stream);
  dim3 grid((unsigned)items, (a.num_kv_heads + kRowsHeads - 1) / kRowsHeads), block(256);
  if (fp8) {
    if (rope) hipLaunchKernelGGL((append_local_rows_kernel<true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((append_local_rows_kernel<true, false>), grid, block, 0, stream, a);
  } else {
    if (rope) hipLaunchKernelGGL((append_local_rows_kernel<false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((append_local_rows_kernel<false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_append_global_rows(const AppendArgs& a, bool compressed, int max_q_len, hipStream_t stream) {
  const int64_t items = rows_items(a, max_q_len);
  if (items == 0) return hipSuccess;
  if (items > 0x7fffffff) return launch_append_global(a, compressed, false, stream);
  dim3 grid((unsigned)items), block(256);
  if (compressed) hipLaunchKernelGGL((append_global_rows_kernel<true>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((append_global_rows_kernel<false>), grid, block, 0, stream, a);
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
