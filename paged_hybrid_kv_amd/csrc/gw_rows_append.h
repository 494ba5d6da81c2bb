// The prompt rows' own tokens of an attention call, appended page by page
// by the tail workgroups of the call's decode kernel (the decode rows'
// tokens are appended by the decode workgroups themselves, and the prompt
// rows' attention runs in the next launch, so it sees them).
//
// pegainfer PR #1012, Description: the prep step rotates K and stores K/V
// with the store type as a parameter; pegainfer "Gemma 4" page, Scheduling:
// prompt rows share the step with the decode rows.
#pragma once

#include "gw_device.h"
#include "gw_kernels.h"
#include "gw_plan.h"

namespace gw {

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
// range) pairs, numbered sequence by sequence (each wave's lanes scan 64
// sequences at a time).  False when item is past the last pair.
__device__ __forceinline__ bool rows_page(const AppendArgs& a, int item, int lane, RowsPage& rp) {
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

// Local family.  K unit (k, t, c) (16 bytes at ((k*16 + t)*4 + c)*16 of the
// K block) holds dims 64c + W k .. + W-1 of slot t (W = 8 bf16 / 16 e4m3);
// quarters c and c + 2 are rotation partners, so thread (t, k, c < 2)
// makes both.  V unit (u, l) (16 bytes at (u*64 + l)*16 of the V block)
// holds dims 4l .. 4l+3 of slots T u .. T u + T-1 (T = 2 bf16 / 4 e4m3).
// A workgroup takes kRowsHeads KV heads of its page: every head's inputs
// are loaded first, in one round trip, and the rotary factors of a slot
// (the same for every head) once.
constexpr int kRowsHeads = kRowsAppendHeads;

// Page item `item`, KV heads h0 .. h0 + kRowsHeads - 1, by 256 threads
// (tid 0 .. 255; all four waves take part).
template <bool FP8, bool ROPE>
__device__ __forceinline__ void append_local_rows_page(const AppendArgs& a, int item, int h0, int tid) {
  constexpr int kW = FP8 ? 16 : 8;           // dims per K unit
  constexpr int kU = FP8 ? 4 : 8;            // K units per quarter
  constexpr int kT = FP8 ? 4 : 2;            // slots per V unit
  constexpr int kVOff = FP8 ? 4096 : 8192;
  constexpr int kVUnits = (kPage / kT) * 64;          // V units per (page, head)
  constexpr int kVPer = (kVUnits + 255) / 256;        // V units per thread
  RowsPage rp;
  if (!rows_page(a, item, tid & 63, rp)) return;
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
// Page item `item` by 256 threads (tid 0 .. 255).  An e4m3 page takes the
// per-token record of the single-token append (global_record_lane, then
// put_global_record_e4m3), one token per wave at a time.
template <bool COMPRESSED, bool FP8>
__device__ __forceinline__ void append_global_rows_page(const AppendArgs& a, int item, int tid) {
  RowsPage rp;
  if (!rows_page(a, item, tid & 63, rp)) return;
  uint8_t* pb = a.pool + (int64_t)rp.page * a.page_bytes;
  if constexpr (FP8) {
    const int w = tid >> 6, l = tid & 63;
    for (int t = rp.t0 + w; t <= rp.t1; t += 4) {
      const uint16_t* vr = a.v + (int64_t)(rp.r0 + rp.pg * kPage + t - rp.p0) * 512;
      const uint16_t* kr = a.k_raw ? a.k_raw + (vr - a.v) : vr;   // the same row of k_raw
      const GlobalRecordLane r = global_record_lane(vr, kr, a.rope_cos, a.rope_sin, rp.pg * kPage + t, l);
      put_global_record_e4m3<COMPRESSED>(pb, r, t, l);
    }
    return;
  }
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

// Argument blocks of the rows append for a call's arguments: the call's
// rows are the tokens, one-row sequences left to the decode workgroups.
__device__ __forceinline__ AppendArgs rows_append_args(const LocalAttnArgs& a) {
  AppendArgs ap{};
  ap.pool = const_cast<uint8_t*>(a.pool);
  ap.page_bytes = a.page_bytes;
  ap.head_bytes = a.head_bytes;
  ap.k_raw = a.k_new;
  ap.v = a.v_new;
  ap.page_table = a.page_table;
  ap.pt_stride = a.pt_stride;
  ap.rope_cos = a.rope_cos;
  ap.rope_sin = a.rope_sin;
  ap.n_tok = a.num_rows;
  ap.num_kv_heads = a.num_kv_heads;
  ap.q_indptr = a.q_indptr;
  ap.seq_lens = a.seq_lens;
  ap.num_seqs = a.num_seqs;
  ap.skip_single = 1;
  return ap;
}

__device__ __forceinline__ AppendArgs rows_append_args(const GlobalAttnArgs& a) {
  AppendArgs ap{};
  ap.pool = const_cast<uint8_t*>(a.pool);
  ap.page_bytes = a.page_bytes;
  ap.head_bytes = (int32_t)a.page_bytes;
  ap.k_raw = a.k_new;
  ap.v = a.v_new;
  ap.page_table = a.page_table;
  ap.pt_stride = a.pt_stride;
  ap.rope_cos = a.rope_cos;
  ap.rope_sin = a.rope_sin;
  ap.n_tok = a.num_rows;
  ap.num_kv_heads = 1;
  ap.q_indptr = a.q_indptr;
  ap.seq_lens = a.seq_lens;
  ap.num_seqs = a.num_seqs;
  ap.skip_single = 1;
  return ap;
}

// Append unit u of a local call (unit = page item x block of kRowsHeads KV
// heads, the head block fastest), by 256 threads.
template <bool FP8>
__device__ __forceinline__ void local_rows_append_unit(const LocalAttnArgs& a, int u, int tid) {
  const int hblocks = (a.num_kv_heads + kRowsHeads - 1) / kRowsHeads;
  if (u >= a.append_units) return;
  const AppendArgs ap = rows_append_args(a);
  const int item = u / hblocks, h0 = (u % hblocks) * kRowsHeads;
  if (a.rope_cos) append_local_rows_page<FP8, true>(ap, item, h0, tid);
  else append_local_rows_page<FP8, false>(ap, item, h0, tid);
}

// Append unit u (one page item) of a global call, by 256 threads.
template <bool COMPRESSED, bool FP8>
__device__ __forceinline__ void global_rows_append_unit(const GlobalAttnArgs& a, int u, int tid) {
  if (u >= a.append_units) return;
  append_global_rows_page<COMPRESSED, FP8>(rows_append_args(a), u, tid);
}

}  // namespace gw
