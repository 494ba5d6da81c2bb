// Device helpers shared by the gw kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gw {

constexpr int kPage = 16;        // tokens per page, both families
constexpr int kWave = 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 1/ln(2): softmax runs in base 2, z = s * scale * log2(e).
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bits_to_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f32_to_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// bf16 pair (low half = first element) -> two floats, exactly.
__device__ __forceinline__ float bf16_lo(uint32_t p) { return bits_to_f32(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return bits_to_f32(p & 0xffff0000u); }

// Two floats -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// acc + a.lo*b.lo + a.hi*b.hi on bf16 pairs, fp32 accumulate (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), acc, false);
}

// Two e4m3 bytes of a dword (word 0: bytes 0,1; word 1: bytes 2,3) -> packed
// bf16 pair, exactly (every e4m3 value is a bf16 value).
template <bool kHiWord>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHiWord);
  return __builtin_bit_cast(uint32_t, b);
}

// fp32 (already a bf16 value) -> e4m3 code: nearest even, saturating to
// +-448, NaN -> 0x7f | sign.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t u = f32_to_bits(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 24) & 0x80u) | 0x7fu;
  float c = fminf(fmaxf(x, -448.0f), 448.0f);
  int packed = __builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false);
  return (uint32_t)packed & 0xffu;
}

// Round a float to bf16 and back (nearest even), as the stores do.
__device__ __forceinline__ float round_bf16(float x) {
  return bf16_lo(pack_bf16(x, 0.0f));
}

// One rotate-half RoPE pair in fp32 with the rounding fixed by explicit
// fused multiply-adds, so every kernel that rotates K gets the same bits:
//   ya = xa*c - xb*s,  yb = xb*c + xa*s.
__device__ __forceinline__ void rope_pair(float xa, float xb, float c, float s, float& ya, float& yb) {
  ya = __builtin_fmaf(xa, c, -(xb * s));
  yb = __builtin_fmaf(xb, c, xa * s);
}

// Cross-lane moves.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return bits_to_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f32_to_bits(x), kCtrl, 0xf, 0xf, false));
}
constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;    // row_ror:4  (within 16-lane rows)
constexpr int kRowRor8 = 0x128;    // row_ror:8
constexpr int kRowShl4 = 0x104;    // row_shl:4: lane i reads lane i + 4 of its row

// Max over the 64 lanes of a value held identically by the 4 lanes of each
// quad and differing across quads: two DPP rotations inside each 16-lane
// row, then the four row results through SGPRs.  Returns a wave-uniform value.
__device__ __forceinline__ float wave_max_quads(float x) {
  x = fmaxf(x, bits_to_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f32_to_bits(x), kRowRor4, 0xf, 0xf, false)));
  x = fmaxf(x, bits_to_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f32_to_bits(x), kRowRor8, 0xf, 0xf, false)));
  const float r0 = bits_to_f32((uint32_t)__builtin_amdgcn_readlane((int)f32_to_bits(x), 0));
  const float r1 = bits_to_f32((uint32_t)__builtin_amdgcn_readlane((int)f32_to_bits(x), 16));
  const float r2 = bits_to_f32((uint32_t)__builtin_amdgcn_readlane((int)f32_to_bits(x), 32));
  const float r3 = bits_to_f32((uint32_t)__builtin_amdgcn_readlane((int)f32_to_bits(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ float shfl_xor_f32(float x, int m) {
  return bits_to_f32((uint32_t)__shfl_xor((int)f32_to_bits(x), m, kWave));
}
__device__ __forceinline__ float shfl_down_f32(float x, int d) {
  return bits_to_f32((uint32_t)__shfl_down((int)f32_to_bits(x), d, kWave));
}
__device__ __forceinline__ uint32_t readlane_u32(uint32_t x, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, lane);
}
__device__ __forceinline__ int uniform_i32(int x) { return __builtin_amdgcn_readfirstlane(x); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Streaming 16-byte load (KV pages are read once per call).
__device__ __forceinline__ uint4 ld16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ uint4 ld16_cached(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Wait until every memory access this wave issued has completed (on gfx9
// stores are counted in vmcnt): s_waitcnt vmcnt(0), expcnt/lgkmcnt untouched.
// The signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void wait_stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Event times of the trace build (compiled with GW_TRACE; nothing otherwise):
// workgroup b records event k at trace[16 b + k], in ticks of the 100 MHz
// constant clock (s_memrealtime), or a value (GW_TRACE_V).  The slots each
// kernel uses are listed where it records them; paged_hybrid_kv_amd/trace.py
// reads them back.
#ifdef GW_TRACE
#define GW_TRACE_T(args, k, cond)                                                                         \
  do {                                                                                                   \
    if ((args).trace && (cond)) (args).trace[16 * (int64_t)blockIdx.x + (k)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define GW_TRACE_V(args, k, cond, val)                                                 \
  do {                                                                                \
    if ((args).trace && (cond)) (args).trace[16 * (int64_t)blockIdx.x + (k)] = (uint64_t)(val); \
  } while (0)
// the same at trace row `row` (kernels that share a call's buffer with
// another kernel record at rows of their own)
#define GW_TRACE_AT(args, row, k, cond)                                                                  \
  do {                                                                                                   \
    if ((args).trace && (cond)) (args).trace[16 * (int64_t)(row) + (k)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define GW_TRACE_VAT(args, row, k, cond, val)                                        \
  do {                                                                              \
    if ((args).trace && (cond)) (args).trace[16 * (int64_t)(row) + (k)] = (uint64_t)(val); \
  } while (0)
// the XCD (XCC_ID hardware register, bits 3:0) the workgroup runs on
#define GW_TRACE_XCC() ((uint64_t)__builtin_amdgcn_s_getreg((3 << 11) | 20))
#else
#define GW_TRACE_T(args, k, cond) \
  do {                            \
  } while (0)
#define GW_TRACE_V(args, k, cond, val) \
  do {                                 \
  } while (0)
#define GW_TRACE_AT(args, row, k, cond) \
  do {                                  \
  } while (0)
#define GW_TRACE_VAT(args, row, k, cond, val) \
  do {                                        \
  } while (0)
#define GW_TRACE_XCC() 0ull
#endif
// first trace row of the prompt-row kernels (the decode kernels of the same
// call record at rows 0 .. grid - 1)
constexpr int kTracePrefillRow = 4096;

// Reductions over the lanes l, l^16, l^32, l^48 (the four lanes holding one
// MFMA 16x16 column): v_permlane32_swap / v_permlane16_swap exchange the
// halves / the 16-lane rows of a register with itself, so each step pairs a
// lane with its xor-32 / xor-16 partner without going through LDS.  The
// result is the same in all four lanes.
__device__ __forceinline__ float max_lanes_xor16_32(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(f32_to_bits(x), f32_to_bits(x), false, false);
  x = fmaxf(bits_to_f32((uint32_t)a[0]), bits_to_f32((uint32_t)a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(f32_to_bits(x), f32_to_bits(x), false, false);
  return fmaxf(bits_to_f32((uint32_t)b[0]), bits_to_f32((uint32_t)b[1]));
}
__device__ __forceinline__ float sum_lanes_xor16_32(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(f32_to_bits(x), f32_to_bits(x), false, false);
  x = bits_to_f32((uint32_t)a[0]) + bits_to_f32((uint32_t)a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(f32_to_bits(x), f32_to_bits(x), false, false);
  return bits_to_f32((uint32_t)b[0]) + bits_to_f32((uint32_t)b[1]);
}

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's 16 bytes at gptr land at LDS byte address lds_base + 16 l, where
// lds_base (wave-uniform) goes in M0.  Written as inline assembly so that the
// compiler does not treat every later LDS read as possibly aliasing the
// transfer (it would wait for all outstanding loads before each one); the
// caller waits for completion itself (wait_vmcnt) before a barrier.
__device__ __forceinline__ void dma16_to_lds(const void* gptr, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds_base) : "memory");
}
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
// s_waitcnt vmcnt(N): at most N vector memory operations of this wave left
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Barrier that orders LDS accesses only: outstanding global loads stay in
// flight across it, and the compiler does not move LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wait until at most k groups of this wave's transfers remain in flight, a
// group being kPer transfers (k = groups issued after the one about to be
// read; 0 <= k <= 4).
template <int kPer>
__device__ __forceinline__ void wait_groups_after(int k) {
  switch (k) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<kPer>(); break;
    case 2: wait_vmcnt<2 * kPer>(); break;
    case 3: wait_vmcnt<3 * kPer>(); break;
    default: wait_vmcnt<4 * kPer>(); break;
  }
}

// Physical page ids of a run of n logical pages (pt[0 .. n)), held 64 per
// register, 256 at a time, and read back with readlane, so a page loop that
// streams pages by direct-to-LDS transfers issues no vector memory operation
// the compiler would wait on.  Asking for page i >= base + 256 reloads the
// next 256 (the loads are waited for at once, inside that rare branch, so
// the compiler's wait stays there).  get() must be called with uniform,
// non-decreasing i.
struct PageIds {
  const int32_t* pt;
  int n, base, lane;
  int v0, v1, v2, v3;
  __device__ __forceinline__ void load(int b) {
    base = b;
    v0 = b + lane < n ? pt[b + lane] : 0;
    v1 = b + 64 < n && b + 64 + lane < n ? pt[b + 64 + lane] : 0;
    v2 = b + 128 < n && b + 128 + lane < n ? pt[b + 128 + lane] : 0;
    v3 = b + 192 < n && b + 192 + lane < n ? pt[b + 192 + lane] : 0;
    asm volatile("" ::"v"(v0), "v"(v1), "v"(v2), "v"(v3));
  }
  __device__ __forceinline__ void init(const int32_t* pt_, int n_, int lane_) {
    pt = pt_;
    n = n_;
    lane = lane_;
    load(0);
  }
  __device__ __forceinline__ int get(int i) {
    if (i >= base + 256) load(i & ~255);
    const int k = i - base, l = k & 63;
    return k < 64 ? __builtin_amdgcn_readlane(v0, l)
         : k < 128 ? __builtin_amdgcn_readlane(v1, l)
         : k < 192 ? __builtin_amdgcn_readlane(v2, l)
                   : __builtin_amdgcn_readlane(v3, l);
  }
};

// One token's global-family record, computed by one wave (Gewell post,
// "the Why": K and V are tied and only K's first 128 dims rotate, so the
// record is V plus the rotated quarter of K).  Lane l holds V chunk l (dims
// 8l .. 8l+7, bf16 as given); lanes 0..7 also hold K chunks l and l + 8
// (dims 8l .. and 64 + 8l ..) of ksrc -- V itself when K is V before
// rotation, or the caller's K when it differs there (a norm weight on K) --
// rotated as rotate-half pairs (i, i + 64) by position pos from the fp32
// tables [pos][64], rounded to bf16.
struct GlobalRecordLane {
  uint4 v, ka, kb;
};
__device__ __forceinline__ GlobalRecordLane global_record_lane(const uint16_t* vsrc, const uint16_t* ksrc,
                                                               const float* rope_cos, const float* rope_sin, int pos,
                                                               int l) {
  GlobalRecordLane r;
  r.v = *reinterpret_cast<const uint4*>(vsrc + 8 * l);
  r.ka = r.kb = uint4{0u, 0u, 0u, 0u};
  if (l < 8) {
    const uint4 araw = ksrc == vsrc ? r.v : *reinterpret_cast<const uint4*>(ksrc + 8 * l);
    const uint4 praw = *reinterpret_cast<const uint4*>(ksrc + 64 + 8 * l);
    const uint32_t xa_p[4] = {araw.x, araw.y, araw.z, araw.w};
    const uint32_t xb_p[4] = {praw.x, praw.y, praw.z, praw.w};
    const float* cp = rope_cos + (int64_t)pos * 64 + 8 * l;
    const float* sp = rope_sin + (int64_t)pos * 64 + 8 * l;
    uint32_t ya[4], yb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float a0 = bf16_lo(xa_p[m]), a1 = bf16_hi(xa_p[m]);
      const float b0 = bf16_lo(xb_p[m]), b1 = bf16_hi(xb_p[m]);
      float y0a, y0b, y1a, y1b;
      rope_pair(a0, b0, cp[2 * m], sp[2 * m], y0a, y0b);
      rope_pair(a1, b1, cp[2 * m + 1], sp[2 * m + 1], y1a, y1b);
      ya[m] = pack_bf16(y0a, y1a);
      yb[m] = pack_bf16(y0b, y1b);
    }
    r.ka = uint4{ya[0], ya[1], ya[2], ya[3]};
    r.kb = uint4{yb[0], yb[1], yb[2], yb[3]};
  }
  return r;
}

// Store a token's record (global_record_lane of lane l) at slot `slot` of a
// global page at pb (pool or LDS copy): compressed page = V[16][512] |
// K_rot[16][128], full page = K[16][512] | V[16][512], blocks chunk-major
// ((c*16 + t)*8 + e).
template <bool COMPRESSED>
__device__ __forceinline__ void put_global_record(uint8_t* pb, const GlobalRecordLane& r, int slot, int l) {
  uint8_t* vblock = COMPRESSED ? pb : pb + 16384;
  uint8_t* kblock = COMPRESSED ? pb + 16384 : pb;
  *reinterpret_cast<uint4*>(vblock + (l * 16 + slot) * 16) = r.v;
  // K chunk l: the rotated chunk (l < 8) or, in the full record, V's (K dims
  // >= 128 are V's); the value is selected, not the source, so the record
  // stays in registers
  const bool rot = l < 8;
  if (rot || (!COMPRESSED && l >= 16)) {
    const uint4 k = {rot ? r.ka.x : r.v.x, rot ? r.ka.y : r.v.y, rot ? r.ka.z : r.v.z, rot ? r.ka.w : r.v.w};
    *reinterpret_cast<uint4*>(kblock + (l * 16 + slot) * 16) = k;
  }
  if (rot) *reinterpret_cast<uint4*>(kblock + ((l + 8) * 16 + slot) * 16) = r.kb;
}

// Eight bf16 (a 16-byte chunk) -> their eight e4m3 codes, in order.
__device__ __forceinline__ uint2 e4m3x8_of_bf16x8(const uint4& c) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t b[8];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    b[2 * m] = f32_to_e4m3(bf16_lo(w[m]));
    b[2 * m + 1] = f32_to_e4m3(bf16_hi(w[m]));
  }
  return uint2{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
}

// The same record in an e4m3 global page: each element is the e4m3 code of
// its bf16 value; compressed page = V[16][512] | K_rot[16][128], full page =
// K[16][512] | V[16][512], blocks chunk-major with 16-dim chunks
// ((c*16 + t)*16 + e): lane l's 8 dims are half (l & 1) of chunk l / 2.
template <bool COMPRESSED>
__device__ __forceinline__ void put_global_record_e4m3(uint8_t* pb, const GlobalRecordLane& r, int slot, int l) {
  uint8_t* vblock = COMPRESSED ? pb : pb + 8192;
  uint8_t* kblock = COMPRESSED ? pb + 8192 : pb;
  auto at = [&](uint8_t* blk, int c8) { return blk + ((c8 >> 1) * 16 + slot) * 16 + 8 * (c8 & 1); };
  const uint2 v8 = e4m3x8_of_bf16x8(r.v);
  *reinterpret_cast<uint2*>(at(vblock, l)) = v8;
  const bool rot = l < 8;   // as in put_global_record: select the value, not the source
  if (rot || (!COMPRESSED && l >= 16)) {
    const uint2 ka8 = e4m3x8_of_bf16x8(r.ka);
    const uint2 k = {rot ? ka8.x : v8.x, rot ? ka8.y : v8.y};
    *reinterpret_cast<uint2*>(at(kblock, l)) = k;
  }
  if (rot) *reinterpret_cast<uint2*>(at(kblock, l + 8)) = e4m3x8_of_bf16x8(r.kb);
}

template <bool COMPRESSED, bool FP8>
__device__ __forceinline__ void put_global_record_as(uint8_t* pb, const GlobalRecordLane& r, int slot, int l) {
  if constexpr (FP8) put_global_record_e4m3<COMPRESSED>(pb, r, slot, l);
  else put_global_record<COMPRESSED>(pb, r, slot, l);
}

}  // namespace gw

namespace gw {

// Sum / max over the 64 lanes of a wave, by DPP moves (no LDS round
// trips): inclusive prefixes within each 16-lane row (row_shr 1, 2, 4, 8),
// then lane 15 of rows 0 and 2 into rows 1 and 3 (row_bcast:15) and lane 31
// into rows 2 and 3 (row_bcast:31); lane 63 ends with the whole wave's
// value.  A lane a move does not reach takes 0, which neither changes a sum
// nor, for values >= 0, a max (wave_max_nonneg_i32 takes only such values).
__device__ __forceinline__ int wave_sum_i32(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31, rows 2 and 3
  return __builtin_amdgcn_readlane(x, 63);
}

__device__ __forceinline__ int wave_max_nonneg_i32(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(x, 63);
}

// Prompt-row work items of an attention call.  The prompt sequences (more
// than one query row) are cut into groups of `rows` consecutive rows, and
// the groups are numbered level by level: level k holds, in sequence order,
// the k-th last group of every prompt sequence that has more than k groups.
// A later group of a sequence attends a longer key range, so the items with
// the longest ranges of all sequences are dispatched first and the shorter
// ones fill in behind them as workgroups finish.
struct PromptItem {
  int s;       // sequence
  int grp;     // row group (rows grp * rows ..), counted from the sequence's first row
  int row0;    // the sequence's first row in the call
  int q_len;   // its rows in the call
  int len;     // its length, the call's tokens included
};

// Sequences held in registers, 64 per chunk; a call with more reads the
// rest again on every pass.
constexpr int kPromptItemChunks = 4;

// Item `item` (uniform) of the call; false past the last.  Every lane of the
// wave must take part.
__device__ inline bool prompt_item(const int32_t* q_indptr, const int32_t* seq_lens, int num_seqs, int rows,
                                   int item, int lane, PromptItem& it) {
  constexpr int kC = kPromptItemChunks;
  auto load = [&](int c0, int& o_cnt, int& o_row0, int& o_qlen, int& o_len) __attribute__((always_inline)) {
    const int sl = c0 + lane;
    o_cnt = o_row0 = o_qlen = o_len = 0;
    if (sl < num_seqs) {
      o_row0 = q_indptr[sl];
      o_qlen = q_indptr[sl + 1] - o_row0;
      o_len = seq_lens[sl];
      if (o_qlen > 1) o_cnt = (o_qlen + rows - 1) / rows;
    }
  };
  int cnt[kC], r0[kC], ql[kC], ln[kC];
#pragma unroll
  for (int c = 0; c < kC; ++c) load(64 * c, cnt[c], r0[c], ql[c], ln[c]);
  // items in the levels below k: sum over sequences of min(groups, k)
  auto count_below = [&](int k) __attribute__((always_inline)) {
    int t = 0;
#pragma unroll
    for (int c = 0; c < kC; ++c) t += min(cnt[c], k);
    for (int c0 = 64 * kC; c0 < num_seqs; c0 += 64) {
      int cn, a, b, d;
      load(c0, cn, a, b, d);
      t += min(cn, k);
    }
    return wave_sum_i32(t);
  };
  int mx = 0;
#pragma unroll
  for (int c = 0; c < kC; ++c) mx = max(mx, cnt[c]);
  for (int c0 = 64 * kC; c0 < num_seqs; c0 += 64) {
    int cn, a, b, d;
    load(c0, cn, a, b, d);
    mx = max(mx, cn);
  }
  const int levels = wave_max_nonneg_i32(mx);
  if (item < 0 || item >= count_below(levels)) return false;
  // the item's level k: count_below(k) <= item < count_below(k + 1)
  int lo = 0, hi = levels;   // count_below(lo) <= item < count_below(hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (count_below(mid) <= item) lo = mid;
    else hi = mid;
  }
  const int k = lo;
  int r = item - count_below(k);   // rank of the item's sequence among those with more than k groups
  auto pick = [&](uint64_t m, int c0, int cn, int rr, int qq, int ll) __attribute__((always_inline)) {
    const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    const uint64_t hit = __ballot(((m >> lane) & 1) && rank == r);
    if (hit == 0) return false;   // r < popcount(m) makes this unreachable
    const int ls = __builtin_ctzll(hit);
    it.s = c0 + ls;
    it.grp = __builtin_amdgcn_readlane(cn, ls) - 1 - k;
    it.row0 = __builtin_amdgcn_readlane(rr, ls);
    it.q_len = __builtin_amdgcn_readlane(qq, ls);
    it.len = __builtin_amdgcn_readlane(ll, ls);
    return true;
  };
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const uint64_t m = __ballot(cnt[c] > k);
    const int p = __popcll(m);
    if (r < p) return pick(m, 64 * c, cnt[c], r0[c], ql[c], ln[c]);
    r -= p;
  }
  for (int c0 = 64 * kC; c0 < num_seqs; c0 += 64) {   // ends: the item exists
    int cn, rr, qq, ll;
    load(c0, cn, rr, qq, ll);
    const uint64_t m = __ballot(cn > k);
    const int p = __popcll(m);
    if (r < p) return pick(m, c0, cn, rr, qq, ll);
    r -= p;
  }
  return false;
}

}  // namespace gw
