// Kernel templates of the split decode (decode.hip describes the design),
// included by the four sources that instantiate its variants: decode.hip
// (contiguous cache), decode_paged.hip (paged cache), decode_rot.hip and
// decode_paged_rot.hip (rotated caches).
#pragma once
#include <math.h>

#include <hip/hip_ext.h>

#include <type_traits>

#include "foscar_internal.h"

namespace foscar {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;

// Optional per-work-group timeline, compiled in only with -DFOSCAR_TIMELINE
// (a separate library, libfoscar_timeline.so, built by `build --timeline`;
// the default build compiles every mark to nothing).  Thread 0 of a
// work-group records s_memrealtime (100 MHz) per work item: 0 item start,
// 1 query prologue done, 2 tile loop done, 3 hand-off done, 4 item end; slot
// 5 holds the item (b << 40 | pair << 20 | range), 6 is 1 for the work-group
// that merged, 7 the hardware id (XCC id << 32 | HW_ID).
#ifdef FOSCAR_TIMELINE
constexpr int kTimelineWgs = 8192, kTimelineItems = 8;
__device__ unsigned long long g_timeline[kTimelineWgs][kTimelineItems][8];
__shared__ int s_timeline_item;  // the work-group's item number: an LDS read never waits for loads in flight
__device__ __forceinline__ unsigned timeline_wg() { return blockIdx.x + gridDim.x * blockIdx.y; }
__device__ __forceinline__ void timeline_item(int it) {
  if (threadIdx.x == 0) s_timeline_item = it;
}
__device__ __forceinline__ void timeline_set(int k, unsigned long long v) {
  const unsigned wg = timeline_wg();
  if (threadIdx.x == 0 && wg < kTimelineWgs) {
    const int it = s_timeline_item;
    if (it >= 0 && it < kTimelineItems) g_timeline[wg][it][k] = v;
  }
}
__device__ __forceinline__ void timeline_mark(int k) { timeline_set(k, __builtin_amdgcn_s_memrealtime()); }
__device__ __forceinline__ void timeline_hw() {
  timeline_set(7, (unsigned long long)__builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (15 << 11)) << 32 |
                      __builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11)));
}
#else
__device__ __forceinline__ void timeline_item(int) {}
__device__ __forceinline__ void timeline_set(int, unsigned long long) {}
__device__ __forceinline__ void timeline_mark(int) {}
__device__ __forceinline__ void timeline_hw() {}
#endif

__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t e) { return (x & m) | e; }
__device__ __forceinline__ h4 cat4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(h4, (unsigned long long)lo | ((unsigned long long)hi << 32));
}
__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float half_lo(uint32_t u) { return (float)__builtin_bit_cast(h2, u)[0]; }
__device__ __forceinline__ float half_hi(uint32_t u) { return (float)__builtin_bit_cast(h2, u)[1]; }
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  h2 v = {(_Float16)lo, (_Float16)hi};
  return as_u32(v);
}
__device__ __forceinline__ uint32_t splat_f16(float c) { return pack_f16(c, c); }
__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Code -> fp16 operand construction.  A packed word holds E codes; element e
// sits at bit bits*(e/2) + 16*(e%2), so pair k = elements (2k, 2k+1) occupies
// the same bit position p_k in both half-words.  AND with the pair's 2-bit
// (4-bit) mask after an optional shift that brings it to position p, OR with
// the fp16 exponent that gives mantissa bit p the weight 1: each half then
// reads exactly C + code with C = 2^(10 - p).
// ---------------------------------------------------------------------------
template <int BITS>
struct Codec;

template <>
struct Codec<2> {
  static constexpr int E = 16;      // codes per word
  static constexpr int PAIRS = 8;   // fp16 pairs per word
  static constexpr int NCONST = 6;
  // C of pair k (positions 4, 6, 8 -> 64, 16, 4)
  __host__ __device__ static constexpr float bias(int k) {
    return (k == 4 || k == 7) ? 4.0f : ((k == 1 || k == 3 || k == 6) ? 16.0f : 64.0f);
  }
  // masks and exponent words; kept in registers so that each pair is one v_and_or_b32
  static constexpr uint32_t kConst[NCONST] = {0x00300030u, 0x00C000C0u, 0x03000300u,
                                              0x54005400u, 0x4C004C00u, 0x44004400u};
  __device__ static __forceinline__ void extract(uint32_t w, const uint32_t (&k)[NCONST], uint32_t (&p)[8]) {
    const uint32_t l = w << 4, r = w >> 6;
    p[0] = and_or(l, k[0], k[3]);  // bits 0-1   -> 4-5, C = 64
    p[1] = and_or(l, k[1], k[4]);  // bits 2-3   -> 6-7, C = 16
    p[2] = and_or(w, k[0], k[3]);  // bits 4-5
    p[3] = and_or(w, k[1], k[4]);  // bits 6-7
    p[4] = and_or(w, k[2], k[5]);  // bits 8-9,        C = 4
    p[5] = and_or(r, k[0], k[3]);  // bits 10-11 -> 4-5
    p[6] = and_or(r, k[1], k[4]);  // bits 12-13 -> 6-7
    p[7] = and_or(r, k[2], k[5]);  // bits 14-15 -> 8-9
  }
};

template <>
struct Codec<4> {
  static constexpr int E = 8;
  static constexpr int PAIRS = 4;
  static constexpr int NCONST = 2;
  __host__ __device__ static constexpr float bias(int) { return 64.0f; }
  static constexpr uint32_t kConst[NCONST] = {0x00F000F0u, 0x54005400u};
  __device__ static __forceinline__ void extract(uint32_t w, const uint32_t (&k)[NCONST], uint32_t (&p)[4]) {
    p[0] = and_or(w << 4, k[0], k[1]);  // bits 0-3   -> 4-7, C = 64
    p[1] = and_or(w, k[0], k[1]);       // bits 4-7
    p[2] = and_or(w >> 4, k[0], k[1]);  // bits 8-11  -> 4-7
    p[3] = and_or(w >> 8, k[0], k[1]);  // bits 12-15 -> 4-7
  }
};

// ---------------------------------------------------------------------------
// Key operands of the block-scaled matrix cores (v_mfma_scale_f32_16x16x128_
// f8f6f4) for token-wise keys.  Facts measured on gfx950 with in-bounds
// probes (one-hot operands):
//   * an INT2 code under the mask 0x33333333 is an fp4 (e2m1) nibble 00qq,
//     exactly q/2; an INT4 code under 0x0F0F0F0F an fp8 (e4m3) byte, exactly
//     q * 2^-9; the E8M0 operand scale 2 (2^9) restores q.  One AND per
//     register, a shift for every other one: no per-value convert, no bias;
//   * K slots: an fp4 operand's lane group g, nibble e meets lane group
//     2(g%2) + e/16, byte 16(g/2) + e%16 of an 8-bit operand; two 8-bit
//     operands meet at the same lane group and byte;
//   * the E8M0 scale of 32-element block kb (supplied by lane group kb of the
//     scale register) applies to byte b of lane group G of an 8-bit operand
//     when kb = 2(b/16) + G/2, so per-row scales are the safe form;
//   * products are summed with about 14 significant bits relative to the
//     largest product of each group of 8 (and group sums likewise): fine for
//     query x key code products, whose range is bounded, but not for softmax
//     weights spanning more than 2^14, so P V stays on the fp16 path.
// A key tile of 64 tokens is 4 blocks of 16: block j, column n is token
// 4n + j, so each lane of the result holds one query head's scores for the
// 4 tokens of one quad, as the fp16 P V path expects.
// ---------------------------------------------------------------------------
typedef int v8i __attribute__((ext_vector_type(8)));

template <int BITS>
struct MxKey;
template <>
struct MxKey<2> {
  static constexpr int FMT = 4;           // fp4 e2m1 (cbsz / blgp code)
  static constexpr int CODE_SCALE = 128;  // E8M0 2^1: q/2 -> q
  static constexpr int WPL = 2;           // packed words per lane per block
  __device__ static __forceinline__ v8i build(const uint32_t* w) {
    const uint32_t M = 0x33333333u;
    v8i r;
    r[0] = (int)(w[0] & M);
    r[1] = (int)((w[0] >> 2) & M);
    r[2] = (int)(w[1] & M);
    r[3] = (int)((w[1] >> 2) & M);
    r[4] = r[5] = r[6] = r[7] = 0;
    return r;
  }
  // key channel that byte b of lane group G of the query operand meets (lane
  // group g of the key operand holds channels 32g .. 32g+31 in words 2g, 2g+1)
  __host__ __device__ static constexpr int chan(int G, int b) {
    return 64 * (b >> 4) + 16 * G + 4 * (b & 3) + ((b >> 2) & 3);
  }
  // lane group G's channels in local order l: 16G + l (l < 16), 64 + 16G + l - 16; byte b is
  // local value local(b), and the 16-byte chunk i of the local values is chunk quad_index(G, i)
  // of the query row
  __host__ __device__ static constexpr int local(int b) { return 16 * (b >> 4) + 4 * (b & 3) + ((b >> 2) & 3); }
  __host__ __device__ static constexpr int quad_index(int G, int i) { return 2 * G + (i < 2 ? i : 6 + i); }
};
template <>
struct MxKey<4> {
  static constexpr int FMT = 0;           // fp8 e4m3
  static constexpr int CODE_SCALE = 136;  // E8M0 2^9: q * 2^-9 -> q
  static constexpr int WPL = 4;
  __device__ static __forceinline__ v8i build(const uint32_t* w) {
    const uint32_t M = 0x0F0F0F0Fu;
    v8i r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[2 * i] = (int)(w[i] & M);
      r[2 * i + 1] = (int)((w[i] >> 4) & M);
    }
    return r;
  }
  __host__ __device__ static constexpr int chan(int G, int b) {
    return 32 * G + 8 * (b >> 3) + 4 * (b & 1) + ((b >> 1) & 3);
  }
  // lane group G's channels in local order l: 32G + l
  __host__ __device__ static constexpr int local(int b) { return 8 * (b >> 3) + 4 * (b & 1) + ((b >> 1) & 3); }
  __host__ __device__ static constexpr int quad_index(int G, int i) { return 4 * G + i; }
};

template <int AFMT, int BFMT>
__device__ __forceinline__ f4 mx_mma(const v8i& a, const v8i& b, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f4{0.f, 0.f, 0.f, 0.f}, AFMT, BFMT, 0, sa, 0, sb);
}

// ---------------------------------------------------------------------------
// LDS staging.  Tiles arrive in LDS by global_load_lds (direct HBM -> LDS, no
// registers held while in flight).  The compiler cannot tell the stages of the
// ring apart and would wait for every such load before any LDS read, so the
// reads of a staged tile are inline asm and this code places the waits itself:
// vmcnt(n) for "all but the last n loads issued have landed", then
// lgkmcnt(0) before the registers are used (touch() makes every later use
// depend on that wait).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)p;
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
template <int OFF>
__device__ __forceinline__ uint4 lds_b128(uint32_t a) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFF) : "memory");
  return make_uint4(v[0], v[1], v[2], v[3]);
}
template <int OFF>
__device__ __forceinline__ uint32_t lds_b32(uint32_t a) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFF) : "memory");
  return v;
}
template <int OFF>
__device__ __forceinline__ uint2 lds_b64(uint32_t a) {
  u32x2 v;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFF) : "memory");
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ void touch(uint32_t& v) { asm volatile("" : "+v"(v)); }
// whole register tuples: a 32-bit asm operand taken from a live tuple costs a copy
__device__ __forceinline__ void touch(uint4& v) {
  u32x4 t = {v.x, v.y, v.z, v.w};
  asm volatile("" : "+v"(t));
  v = make_uint4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void touch(uint2& v) {
  u32x2 t = {v.x, v.y};
  asm volatile("" : "+v"(t));
  v = make_uint2(t[0], t[1]);
}
// Buffer resource over `bytes` bytes at p (raw, unswizzled).  Loads past the
// end read zero, so a tile that runs past the cache capacity stays in bounds.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
// HBM -> LDS: each lane's 16 (4) bytes at voff + soff land at l + 16 (4) * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_u8*)l, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_u8*)l, 4, voff, soff, 0, 0);
}

// Bytes of one staged tile and its layout:
//   [ks | kz | vs | vz (token-wise sides)][K (s | z) rows | V (s | z) rows (channel-wise sides)][K rows][V words].
// A channel-wise side stages the (s, z) rows (256 B each) of the groups the
// tile touches (two for g = 32; for g = 128 both tiles of a unit carry them).
// Scales are loaded in 256-byte blocks (one dword per lane).  A side with one
// group per token has 128 bytes per tile, so the upper half of its block lands
// on the next region; loads into one wave's LDS complete in issue order, so
// issuing the scale blocks first and the K rows after them leaves every region
// holding its own data.
template <int BITS, bool KCH, bool VCH, int GRP>
struct Stage {
  static constexpr int E = 32 / BITS;
  static constexpr int KW = kHeadDim / E;            // key words per token
  static constexpr int VW = kTile / E;               // value token-words per tile
  static constexpr int NGK = KCH ? 0 : kHeadDim / GRP;
  static constexpr int NGV = VCH ? 0 : kHeadDim / GRP;
  static constexpr int KSB = 128 * NGK;              // bytes of ks (equally kz) per tile
  static constexpr int VSB = 128 * NGV;
  static constexpr int NGT = (GRP < kTile) ? kTile / GRP : 1;  // channel-wise groups one tile touches
  static constexpr int KCB = KCH ? 512 * NGT : 0;    // channel-wise K: s rows then z rows
  static constexpr int VCB = VCH ? 512 * NGT : 0;
  static constexpr int SOFF = 0;
  static constexpr int VSOFF = SOFF + 2 * KSB;
  static constexpr int KCOFF = VSOFF + 2 * VSB;
  static constexpr int VCOFF = KCOFF + KCB;
  static constexpr int KOFF = VCOFF + VCB;
  static constexpr int KBYTES = KW * 4 * kTile;      // KW/4 chunks of 1 KB
  static constexpr int VOFF = KOFF + KBYTES;
  static constexpr int VBYTES = VW * kHeadDim * 4;   // VW/2 chunks of 1 KB
  static constexpr int BYTES = VOFF + VBYTES;
  static constexpr int KSL = (KSB + 255) / 256;      // 256-byte scale loads per array
  static constexpr int VSL = (VSB + 255) / 256;
  static constexpr int LOADS = KW / 4 + VW / 2 + 2 * KSL + 2 * VSL + (KCB + VCB) / 256;  // loads per tile
  static_assert(KOFF % 16 == 0, "K rows need 16-byte alignment");
  // ring depth: one staged tile per wave.  A tile is copied into registers
  // before it is processed and its slot refilled at once, so the next tile's
  // load still overlaps the current tile's work; a second slot only halved the
  // work-groups LDS lets a CU hold (the INT4 channel-wise rings took 72 KB: one
  // work-group per CU).  Measured against two slots: INT4 channel-wise
  // 100 -> 66 us per step, long-context INT2 64.0 -> 62.0, the others equal or
  // a few percent faster.
#ifdef FOSCAR_RING_DEPTH
  static constexpr int NS = FOSCAR_RING_DEPTH;
#else
  static constexpr int NS = 1;
#endif
};

// A value the compiler must keep in a VGPR (no literal folding).
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Cross-lane helpers.  Lane l holds query head (l & 3) of quad (l >> 2); the
// lanes of one query head are l, l^4, l^8, ... (stride 4).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// value of lane (l & ~3) | I, i.e. query head I of this lane's quad
template <int I>
__device__ __forceinline__ float quad_bcast(float v) {
  return dpp<(I | (I << 2) | (I << 4) | (I << 6))>(v);
}
// {v of this lane's counterpart in half-wave 0, in half-wave 1}: v_permlane32_swap
// leaves the lower half's values in every lane of its first operand and the
// upper half's in every lane of its second
__device__ __forceinline__ void halves(float v, float& h0, float& h1) {
  float a = v, b = v;
  asm volatile("s_nop 2\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  h0 = a;
  h1 = b;
}
// max over rows (0,1) and (2,3) of 16 lanes: v_permlane16_swap trades the odd
// rows of its first operand with the even rows of its second.
//
// Wait states of the inline-asm cross-lane reads.  A DPP or permlane read of a
// VGPR needs two wait states after an ordinary VALU write of it and three
// after a v_dot2 write (measured on gfx950: with two, a DPP read after
// v_dot2c_f32_f16 returns the register's previous value).  The compiler does
// not insert them before the operands of inline asm, so every block opens
// with three (s_nop 2); reads inside a block follow a plain VALU write and
// take two (s_nop 1).
__device__ __forceinline__ float max_row_pairs(float v) {
  float a = v, b = v;
  asm volatile("s_nop 2\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}
// max over the two half-waves: v_permlane32_swap trades the upper half of its
// first operand with the lower half of its second
__device__ __forceinline__ float max_halves(float v) {
  float a = v, b = v;
  asm volatile("s_nop 2\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}
// max over the lanes of one query head (l, l^4, ..., across the wave), and m:
// the DPP row rotations fused into the max, then the permlane swaps, in one
// block.  Scores are never NaN (masked ones are -inf), so the canonicalising
// max the compiler puts before each cross-lane result is not needed.
__device__ __forceinline__ float wave_max_same_query_and(float v, float m) {
  float a, r;
  asm volatile(
      "s_nop 2\n\t"
      "v_max_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane16_swap_b32 %0, %1\n\t"
      "v_max_f32 %0, %0, %1\n\t"
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %1\n\t"
      "v_max3_f32 %2, %0, %1, %3"
      : "+v"(v), "=&v"(a), "=v"(r)
      : "v"(m));
  return r;
}
// The fp16 pair {fp16(pa * a), fp16(pb * b)}, each product rounded once, where
// a and b are fp16 halves (high when ha / hb) of the words wa and wb.
__device__ __forceinline__ uint32_t mul_f16x2(float pa, uint32_t wa, bool ha, float pb, uint32_t wb, bool hb) {
  uint32_t r;
  if (ha)
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(pa), "v"(wa));
  else
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(pa), "v"(wa));
  if (hb)
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(r) : "v"(pb), "v"(wb));
  else
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "+v"(r) : "v"(pb), "v"(wb));
  return r;
}
// sum over all 64 lanes, in every lane
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0x121>(v);  // row_ror:1
  v += dpp<0x122>(v);  // row_ror:2
  v += dpp<0x124>(v);  // row_ror:4
  v += dpp<0x128>(v);  // row_ror:8
  float a = v, b = v;
  asm volatile("s_nop 2\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  v = a + b;
  a = v;
  b = v;
  asm volatile("s_nop 2\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return a + b;
}
__device__ __forceinline__ float wave_max_same_query(float v) {
  v = fmaxf(v, dpp<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp<0x128>(v));  // row_ror:8
  return max_halves(max_row_pairs(v));
}
// reductions over a row of 16 lanes (the lanes of one query head in the
// block-scaled score layout), with the DPP rotations fused into the operation
// max over the 16 lanes of a row (DPP row rotations), then with m, in one asm block (an fmaxf of
// an asm result and a loop-carried value makes the compiler canonicalise both first: two more
// instructions per tile)
__device__ __forceinline__ float row_max16_and(float v, float m) {
  asm volatile(
      "s_nop 2\n\t"
      "v_max_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_ror:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32 %0, %0, %1"
      : "+v"(v)
      : "v"(m));
  return v;
}
__device__ __forceinline__ float row_sum16(float v) {
  asm volatile(
      "s_nop 2\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:1 row_mask:0xf bank_mask:0xf"
      : "+v"(v));
  return v;
}
// sum over each half-row of 8 lanes: quad swaps, then the half-row mirror
__device__ __forceinline__ float half_row_sum8(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  return v;
}
// v of lane `src` (a wave-uniform lane index), as a scalar operand
__device__ __forceinline__ float lane_value(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// sum over the lanes of one query head within SPAN lanes (32: half-wave, 64: wave),
// with DPP row rotations and v_permlane16/32_swap (no LDS round trip)
template <int SPAN>
__device__ __forceinline__ float sum_same_query(float v) {
  v += dpp<0x124>(v);  // row_ror:4
  v += dpp<0x128>(v);  // row_ror:8
  float a = v, b = v;
  asm volatile("s_nop 2\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  v = a + b;
  if (SPAN == 64) {
    a = v;
    b = v;
    asm volatile("s_nop 2\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    v = a + b;
  }
  return v;
}

template <int N>
__device__ __forceinline__ void load_u2(uint2 (&dst)[N], const uint16_t* p) {
  const uint2* q = reinterpret_cast<const uint2*>(p);
#pragma unroll
  for (int i = 0; i < N; ++i) dst[i] = q[i];
}

// Rotated cache: y = x H for one 128-value row held two values per lane
// (channel 2 lane + e in x_e), H the orthonormal Sylvester-Hadamard matrix
// (entry (i, j) = (-1)^popcount(i & j) / sqrt(128); symmetric, its own
// inverse).  Seven butterfly stages, one per bit of the channel index: bit 0
// inside the lane, bits 1-6 against the lane whose index differs in bit k - 1
// (ds_bpermute); the lower channel of each pair keeps the sum, the upper one
// the difference.  All 64 lanes must run it.
template <typename T>
__device__ __forceinline__ void hadamard_row(T& x0, T& x1, int lane) {
  T s = x0 + x1, d = x0 - x1;
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const T ps = __shfl_xor(s, 1 << k), pd = __shfl_xor(d, 1 << k);
    const bool upper = (lane >> k) & 1;
    s = upper ? ps - s : s + ps;
    d = upper ? pd - d : d + pd;
  }
  const T inv_sqrt128 = (T)0.088388347648318440550;
  x0 = s * inv_sqrt128;
  x1 = d * inv_sqrt128;
}
// bf16 nearest to x, ties to even, for x in fp32's normal range: the fp64
// pattern rounded to 7 stored mantissa bits converts to fp32 exactly
__device__ __forceinline__ uint32_t bf16_rne_f64(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  u += ((uint64_t)1 << 44) - 1 + ((u >> 45) & 1);
  u &= ~(((uint64_t)1 << 45) - 1);
  return __float_as_uint((float)__longlong_as_double((long long)u)) >> 16;
}
// The rotated query: q H of a bf16 pair row (channels 2 lane, 2 lane + 1),
// rounded once to bf16.  The butterflies run in fp64, where the sums of bf16
// values are exact (for rows spanning under 2^38 in magnitude), so the result
// is the bf16 rounding of the exact product up to the fp64 scaling by
// 1/sqrt(128).
__device__ __forceinline__ uint32_t hadamard_bf16_pair(uint32_t w, int lane) {
  double x0 = (double)__uint_as_float(w << 16), x1 = (double)__uint_as_float(w & 0xFFFF0000u);
  hadamard_row(x0, x1, lane);
  return bf16_rne_f64(x0) | (bf16_rne_f64(x1) << 16);
}

// ---------------------------------------------------------------------------
// Split kernel.
// BITS: 2 or 4; KCH / VCH: channel-wise key / value groups; GRP: g.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Fold the S window partials of (row0, channel c0) and (row1, channel c1) into
// running log-sum-exp merges (max m, weighted sum n, weight sum d).
// Device-coherent loads (other work-groups wrote the slots), all issued before
// any is used.  An empty term (lse -inf) adds nothing, and a running max of
// -inf has nothing to rescale.
template <int S>
__device__ __forceinline__ void fold_window_slots(const SplitArgs& a, size_t row0, int c0, size_t row1, int c1,
                                                  float& m0, float& n0, float& d0, float& m1, float& n1, float& d1) {
  constexpr int D = kHeadDim;
  float wl0[S], wl1[S], wo0[S], wo1[S];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    wl0[j] = coherent_load(a.win_lse + row0 * S + j);
    wl1[j] = coherent_load(a.win_lse + row1 * S + j);
    wo0[j] = coherent_load(a.win_o + (row0 * S + j) * D + c0);
    wo1[j] = coherent_load(a.win_o + (row1 * S + j) * D + c1);
  }
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const float b0 = fmaxf(m0, wl0[j]), b1 = fmaxf(m1, wl1[j]);
    const float r0 = (b0 == -INFINITY) ? 1.f : __expf(m0 - b0), r1 = (b1 == -INFINITY) ? 1.f : __expf(m1 - b1);
    const float w0 = (wl0[j] == -INFINITY) ? 0.f : __expf(wl0[j] - b0);
    const float w1 = (wl1[j] == -INFINITY) ? 0.f : __expf(wl1[j] - b1);
    n0 = fmaf(w0, wo0[j], n0 * r0);
    d0 = fmaf(d0, r0, w0);
    n1 = fmaf(w1, wo1[j], n1 * r1);
    d1 = fmaf(d1, r1, w1);
    m0 = b0;
    m1 = b1;
  }
}

// Log-sum-exp merge of the ns ranges of one (sequence, KV head), run by the
// work-group that finished last: O = sum_s exp(lse_s - M) O_s / sum_s exp(lse_s - M),
// lse = M + log(sum_s exp(lse_s - M)).  The partials were written by other
// work-groups, so they are read with device-coherent loads.  Wave i owns query
// row i, lane l its channels 2l and 2l + 1, and the ranges stream in blocks of
// 32 (all of them at the long-context plan): each block's partial outputs
// (64-bit loads, the range in a scalar offset) and lse values (lane u: range
// u) are issued together, one memory round trip per block.  The block's max,
// weights and weight sum are wave reductions, and each weight reaches the
// multiply-adds as a scalar operand (readlane), so the merge needs no LDS and
// no barrier.
// max over all 64 lanes, in every lane (the pattern of wave_sum)
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0x121>(v));  // row_ror:1
  v = fmaxf(v, dpp<0x122>(v));  // row_ror:2
  v = fmaxf(v, dpp<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp<0x128>(v));  // row_ror:8
  float a = v, b = v;
  asm volatile("s_nop 2\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  v = fmaxf(a, b);
  a = v;
  b = v;
  asm volatile("s_nop 2\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}
template <bool ROT>
__device__ __forceinline__ void merge_ranges(const SplitArgs& a, int b, int h, int ns) {
  constexpr int D = kHeadDim, BLK = 32;
  static_assert(kWaves == kMaxG && D == 128, "one wave per query row, two channels per lane");
  const int G = a.g_heads;
  const uint32_t tid = in_vgpr(threadIdx.x);  // opaque: not hoisted out of a work loop
  const int lane = tid & 63;
  const int i = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (i >= G) return;
  const size_t row = (size_t)b * a.hq + (size_t)h * G + i;
  const __amdgpu_buffer_rsrc_t ro = rsrc(a.o_part + row * a.splits * D, (uint32_t)(a.splits * D * 4));
  const uint32_t vo = (uint32_t)lane * 8;
  const float* lp = a.lse_part + row * a.splits;
  float m = -INFINITY, n0 = 0.f, n1 = 0.f, d = 0.f;
  for (int s0 = 0; s0 < ns; s0 += BLK) {
    // unconditional loads (an atomic load under a branch is not speculated, and
    // the branches would serialise the round trips): ranges past ns re-read
    // range ns - 1 and are masked afterwards.  sc1 (cache policy 16): device-
    // coherent, like the relaxed agent-scope atomic loads of the hand-off
    uint2 v[BLK];
#pragma unroll
    for (int u = 0; u < BLK; ++u) {
      const uint32_t so = (uint32_t)(min(s0 + u, ns - 1) * D * 4);
      v[u] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(ro, vo, so, 16));
    }
    const int su = s0 + (lane & (BLK - 1));
    const float l0 = coherent_load(lp + min(su, ns - 1));
    const float l = (lane < BLK && su < ns) ? l0 : -INFINITY;  // every range below ns has a finite lse
    const float bm = fmaxf(m, wave_max(l));
    const float w = __expf(l - bm);  // 0 for masked lanes
    const float r = __expf(m - bm);  // 0 on the first block
    n0 *= r;
    n1 *= r;
    d = fmaf(d, r, wave_sum(w));
#pragma unroll
    for (int u = 0; u < BLK; ++u) {
      const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
      n0 = fmaf(wu, __uint_as_float(v[u].x), n0);  // masked ranges: wu = 0 and a finite re-read
      n1 = fmaf(wu, __uint_as_float(v[u].y), n1);
    }
    m = bm;
  }
  // rotated values: the cache's weighted sum back in the model's basis (the window's rows are in it)
  if (ROT && (a.rot & 2)) hadamard_row(n0, n1, lane);
  // the full-precision window's partials are further terms of the same merge (1, 2, 4 or 8 slots)
  float m1 = m, d1 = d;
  const int c = 2 * lane;
  switch (a.win_wgs) {
    case 1: fold_window_slots<1>(a, row, c, row, c + 1, m, n0, d, m1, n1, d1); break;
    case 2: fold_window_slots<2>(a, row, c, row, c + 1, m, n0, d, m1, n1, d1); break;
    case 4: fold_window_slots<4>(a, row, c, row, c + 1, m, n0, d, m1, n1, d1); break;
    case 8: fold_window_slots<8>(a, row, c, row, c + 1, m, n0, d, m1, n1, d1); break;
    default: break;
  }
  if (!(d > 0.f)) {  // no token at all (no cache range and empty window slots)
    n0 = n1 = 0.f;
    d = 1.f;
    m = -INFINITY;
  }
  const uint32_t packed = (uint32_t)to_bf16_rne(n0 / d) | ((uint32_t)to_bf16_rne(n1 / d) << 16);
  reinterpret_cast<uint32_t*>(a.out + row * D)[lane] = packed;
  if (lane == 0 && a.lse) a.lse[row] = m + __logf(d);
}

// ---------------------------------------------------------------------------
// Work order.  The dispatcher starts work-groups in index order, so the index
// -> (sequence, KV head, range) map decides which work runs last.  With the
// sequence lengths known only on the device, wave 0 of every work-group maps
// its index to a work item, longest first: every full range (all of the same
// length), then the sequences' last partial ranges in eight length buckets,
// longest first, then one item per (empty sequence, KV head) that writes
// out = 0 and lse = -inf.  Work-group indices past the items exit.
// Consecutive indices are different KV heads of one range, which land on
// different XCDs.
// ---------------------------------------------------------------------------
enum : int { kItemRange = 0, kItemEmpty = 1, kItemNone = 2 };

// Inclusive prefix sum over the 64 lanes: Hillis-Steele inside each row of 16
// (DPP row_shr 1, 2, 4, 8 with zero fill), then row_bcast:15 carries row 0's
// total into row 1 and row 2's into row 3, and row_bcast:31 carries the total
// of rows 0-1 into rows 2-3.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_in(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, CTRL < 0x140);
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_in<0x111, 0xf>(v);
  v += dpp_in<0x112, 0xf>(v);
  v += dpp_in<0x114, 0xf>(v);
  v += dpp_in<0x118, 0xf>(v);
  v += dpp_in<0x142, 0xa>(v);
  v += dpp_in<0x143, 0xc>(v);
  return v;
}

// Work classes in dispatch order: full ranges, then each sequence's last
// partial range by length (kPartBuckets buckets, longest first), then empty
// sequences.
constexpr int kPartBuckets = 8;
constexpr int kClasses = 2 + kPartBuckets;

// x / d for 0 <= x <= 2^24 and d >= 1, given r = 1/d rounded to float: the
// float product is within one of x / d, so one correction each way makes the
// truncated quotient exact (d = 1 and 2 have exact reciprocals).
__device__ __forceinline__ int div_u24(int x, int d, float r) {
  int q = (int)((float)x * r);
  const int m = x - q * d;
  q += (m >= d) ? 1 : 0;
  q -= (m < 0) ? 1 : 0;
  return q;
}

// Length granule of the work classes: the tile, or the channel-wise group
// when that is longer (ranges hold whole groups).
template <bool KCH, bool VCH, int GRP>
constexpr int work_unit() { return ((KCH || VCH) && GRP > kTile) ? GRP : kTile; }

struct NextLoad {
  int idx;     // lane 0: the work index
  int tl[16];  // raw lengths of sequences lane * K + k (K = ceil(B / 64)) below B
};
__device__ __forceinline__ void next_load(const SplitArgs& a, NextLoad& n) {
  const int lane = in_vgpr(threadIdx.x) & 63;  // opaque: nothing here is hoisted out of a work loop
  const int B = a.batch, K = (B + 63) / 64;    // sequences per lane, <= 16
  n.idx = 0;
  if (lane == 0) n.idx = __hip_atomic_fetch_add(a.work_ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int bb = lane * K + k;
    n.tl[k] = (k < K && bb < B) ? a.seq_lens[bb] : 0;
  }
}

template <int UNIT>
__device__ __forceinline__ void map_select(const SplitArgs& a, const NextLoad& n, int* item) {
  const int lane = in_vgpr(threadIdx.x) & 63;
  const int K = (a.batch + 63) / 64;
  const int hkv = a.hkv, chunk = a.chunk;
  const int nb = chunk / UNIT;  // units per full range
  const float rc = 1.0f / (float)chunk, rn = 1.0f / (float)nb;
  const int L = __builtin_amdgcn_readfirstlane(n.idx);
  int nf[16], pc[16];  // per sequence: full ranges; class of the last partial range (-1: none, -2: no sequence)
  int cnt[kClasses];   // items of this lane's sequences per class
#pragma unroll
  for (int c = 0; c < kClasses; ++c) cnt[c] = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    nf[k] = 0;
    pc[k] = -2;
    if (!(k < K && lane * K + k < a.batch)) continue;
    const int t = min(max(n.tl[k], 0), a.tcap);
    nf[k] = div_u24(t, chunk, rc);
    const int pu = (t - nf[k] * chunk + UNIT - 1) / UNIT;  // units of the partial range
    pc[k] = (t == 0) ? kClasses - 1 : (pu == 0) ? -1 : kPartBuckets - div_u24((pu - 1) * kPartBuckets, nb, rn);
    cnt[0] += nf[k] * hkv;
#pragma unroll
    for (int c = 1; c < kClasses; ++c) cnt[c] += (pc[k] == c) ? hkv : 0;
  }
  int base = 0, cls = -1, lc = 0, sel = 0;
#pragma unroll
  for (int c = 0; c < kClasses; ++c) {
    const int inc = wave_incl_scan(cnt[c]);
    const int tot = __shfl(inc, 63);
    if (cls < 0 && L < base + tot) {
      cls = c;
      lc = L - base;
      sel = inc - cnt[c];  // this lane's first item in the class
    }
    base += tot;
  }
  if (lane == 0) item[3] = kItemNone;
  if (cls < 0) return;  // uniform: L is past every item
  int run = sel;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if (pc[k] == -2) continue;
    const int m = (cls == 0) ? nf[k] * hkv : (pc[k] == cls) ? hkv : 0;  // items of this sequence in class cls
    if (lc >= run && lc < run + m) {
      const int o = lc - run;
      item[0] = lane * K + k;
      item[1] = o % hkv;
      item[2] = (cls == 0) ? o / hkv : (cls == kClasses - 1) ? 0 : nf[k];
      item[3] = (cls == kClasses - 1) ? kItemEmpty : kItemRange;
      item[4] = min(max(n.tl[k], 0), a.tcap);
    }
    run += m;
  }
}

// The end of a work item: every wave has written its running max m (log2
// units) and denominator l to s_ml and its un-normalised output rows to s_o.
// The work-group merges its 4 waves into this range's (O, lse) and either
// writes the final output (the only range) or stores the partial
// device-coherently and counts its arrival; the last range of the (sequence,
// KV head) merges them all.  Every return is uniform.
template <int UNIT, bool ROT>
__device__ __forceinline__ void finish_range(const SplitArgs& a, const int b, const int h, const int split,
                                             const int T, float (*s_ml)[2][4], float (*s_o)[4][kHeadDim], int* next,
                                             NextLoad& nx) {
  constexpr int D = kHeadDim;
  const uint32_t tid = in_vgpr(threadIdx.x);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t bh = (size_t)b * a.hkv + h;
  const int ns = (T + a.chunk - 1) / a.chunk;  // ranges holding tokens of this sequence
  const bool direct = ns == 1 && !a.win_wgs;  // the only range partial: write the final output
  if (ROT && direct && (a.rot & 2)) {  // rotated values: wave i takes query row i whole, to rotate it back
    const int i = wave, lane = tid & 63;
    if (i < a.g_heads) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[w][0][i]);
      float n0 = 0.f, n1 = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float l = s_ml[w][1][i];
        const float f = (l > 0.f) ? __builtin_amdgcn_exp2f(s_ml[w][0][i] - M) : 0.f;
        n0 = fmaf(f, s_o[w][i][2 * lane], n0);
        n1 = fmaf(f, s_o[w][i][2 * lane + 1], n1);
        den = fmaf(f, l, den);
      }
      hadamard_row(n0, n1, lane);
      const size_t row = (size_t)b * a.hq + h * a.g_heads + i;
      const float o0 = n0 / den, o1 = n1 / den, l_nat = (M + __log2f(den)) * kLn2;
      const uint32_t packed = (uint32_t)to_bf16_rne(o0) | ((uint32_t)to_bf16_rne(o1) << 16);
      reinterpret_cast<uint32_t*>(a.out + row * D)[lane] = packed;
      if (lane == 0 && a.lse) a.lse[row] = l_nat;
    }
    if (next && wave == 0) map_select<UNIT>(a, nx, next);
    return;
  }
  for (int idx = (int)tid; idx < 4 * D; idx += blockDim.x) {
    const int i = idx / D, c = idx % D;
    if (i >= a.g_heads) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[w][0][i]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float l = s_ml[w][1][i];
      const float f = (l > 0.f) ? __builtin_amdgcn_exp2f(s_ml[w][0][i] - M) : 0.f;
      num = fmaf(f, s_o[w][i][c], num);
      den = fmaf(f, l, den);
    }
    const size_t row = (size_t)b * a.hq + h * a.g_heads + i;
    const float o = num / den, l_nat = (M + __log2f(den)) * kLn2;
    if (direct) {  // the only range: final output
      float of = o, lf = l_nat;
      if (a.win_o) {  // merged with the full-precision window's partial
        const float wl = a.win_lse[row];
        const float mm = fmaxf(l_nat, wl), w1 = __expf(l_nat - mm), w2 = __expf(wl - mm);
        of = fmaf(w1, o, w2 * a.win_o[row * D + c]) / (w1 + w2);
        lf = mm + __logf(w1 + w2);
      }
      a.out[row * D + c] = to_bf16_rne(of);
      if (c == 0 && a.lse) a.lse[row] = lf;
    } else {
      // device-coherent stores (they bypass this XCD's L2 for the merging work-group)
      __hip_atomic_store(a.o_part + (row * a.splits + split) * D + c, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (c == 0)
        __hip_atomic_store(a.lse_part + row * a.splits + split, l_nat, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (direct) {
    if (next && wave == 0) map_select<UNIT>(a, nx, next);
    return;
  }

  // ---------------- the last range of this (sequence, KV head) merges all ranges
  // Hand-off without agent-scope fences: those write back and invalidate the
  // whole L2 of the XCD, once per work-group, and serialise the grid's tail.
  // Every value that crosses work-groups is a device-coherent atomic access,
  // so ordering only needs this work-group's stores to have completed
  // (vmcnt 0 in every wave, then the barrier) before the counter increment,
  // and the merging work-group's loads to be issued after it read the count.
  __shared__ int s_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int done = 0;
  if (tid == 0) done = __hip_atomic_fetch_add(a.counters + bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (next && wave == 0) map_select<UNIT>(a, nx, next);  // while the count is in flight
  if (tid == 0) s_last = (done == ns - 1 + a.win_wgs);  // fused window work-groups arrive like ranges
  __syncthreads();
  timeline_mark(3);
  if (!s_last) return;
  merge_ranges<ROT>(a, b, h, ns);
  timeline_set(6, 1);
  if (tid == 0) a.counters[bh] = 0;  // ready for the next call on this workspace
}

// Waves per SIMD the register allocation aims at (the LDS of a one-tile ring
// never limits below it).  INT2 token-wise K and V, g = 128: 4 (128 VGPRs).
// Other INT2 instances: 3 (168 VGPRs): left to themselves they took 180-190
// (2 waves), and 3 waves ran the ragged token-K / channel-V batches 8-11%
// faster and the channel-wise ones 2% faster; token-wise g = 32 would spill.
// INT4: unconstrained; 3 waves made the ragged INT4 batches 2-6% slower.
template <int BITS, bool KCH, bool VCH, int GRP>
constexpr int waves_per_simd() {
  if (BITS == 2 && !KCH && !VCH) return GRP == 128 ? 4 : (GRP == 64 ? 3 : 1);
  return BITS == 2 ? 3 : 1;
}

// One work item: range `split` of KV head h of sequence b (T = 0 and split = 0:
// the empty sequence's rows).  Every return is uniform over the work-group.
// PAGED: the cache is a pool of blocks reached through the block table.
template <int BITS, bool KCH, bool VCH, int GRP, bool PAGED, bool ROT>
__device__ __forceinline__ void run_item(const SplitArgs& a, const int b, const int h, const int split, const int T,
                                         int* next) {
  using C = Codec<BITS>;
  constexpr int D = kHeadDim;
  constexpr int E = C::E;
  constexpr int PAIRS = C::PAIRS;
  constexpr int KPW = PAIRS / 2;           // k-steps (of 4 channels / 4 tokens) per word
  constexpr int QPW = KPW / 2;             // 16-byte operand reads per word (two k-steps each)
  constexpr int KW = D / E;                // key words per token
  constexpr int VW = kTile / E;            // value token-words per tile
  constexpr int NGK = KCH ? 1 : D / GRP;   // key groups per token
  constexpr int NGV = VCH ? 1 : D / GRP;   // value groups per token
  constexpr int UNIT = work_unit<KCH, VCH, GRP>();  // tiles of a range come in whole units
  constexpr int TPU = UNIT / kTile;

  // lane and wave pass through an opaque register: in a persistent loop the
  // compiler would otherwise hoist every per-lane address and constant of the
  // item out of the loop and keep them live through the tile loop
  const uint32_t tid = in_vgpr(threadIdx.x);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r0 = split * a.chunk;
  if (r0 >= T) {  // no token in this range; an empty sequence's rows are written once
    if (T == 0 && split == 0 && !a.win_wgs) {  // (with a window, its work-groups write them)
      for (int idx = (int)tid; idx < a.g_heads * kHeadDim; idx += blockDim.x) {
        const size_t row = (size_t)b * a.hq + h * a.g_heads + idx / kHeadDim;
        a.out[row * kHeadDim + idx % kHeadDim] = 0;  // no token at all: out = 0, lse = -inf
        if (idx % kHeadDim == 0 && a.lse) a.lse[row] = -INFINITY;
      }
    }
    if (next && wave == 0) {
      NextLoad nx;
      next_load(a, nx);
      map_select<UNIT>(a, nx, next);
    }
    return;
  }
  const int r1 = min(r0 + a.chunk, T);

  using ST = Stage<BITS, KCH, VCH, GRP>;
  constexpr int NS = ST::NS;
  extern __shared__ __align__(16) unsigned char smem[];  // kWaves rings of NS staged tiles
  __shared__ uint2 s_p[kWaves][NGV][4][16];   // P operand of (group, query, quad)
  __shared__ float s_ml[kWaves][2][4];        // epilogue: per-wave (m, l) per query
  float (*s_o)[4][D] = reinterpret_cast<float (*)[4][D]>(smem);  // epilogue, reuses the rings

  const int qd = lane >> 2;   // quad: QK block (tokens 4qd..4qd+3); PV block (channels 8qd..8qd+7)
  const int qn = lane & 3;    // QK output column / PV A-operand row = query head within the KV group
  // token-wise keys (block-scaled QK^T): lane 16 rh + rq holds query head rh's scores of tile
  // quad rq; channel-wise keys keep quad qd, head qn.  pq: the quad of this lane's scores
  const int rh = lane >> 4, rq = lane & 15;
  const int pq = KCH ? qd : rq;
  using MK = MxKey<BITS>;
  constexpr int NQM = (!KCH && NGK > 2) ? NGK / 2 : 1;  // block-scaled QK^T instructions per 16 tokens
  const bool qvalid = qn < a.g_heads;
  const size_t bh = (size_t)b * a.hkv + h;
  const float sl2 = a.sm_log2;

  // ---- query prologue: bf16 -> fp16 pairs (channels 2j, 2j+1); exact for values in the fp16 range
  // token-wise K: the work-group's query block as the QK^T B operand in LDS (row = query head;
  // rows padded by 16 B so the four rows of one read fall in different banks), and per group
  // sigma' * sum(Q) and sigma' * sum(Q * C)  (C = operand bias of each channel)
  // channel-wise K: the bf16 query pairs (row = query head) from which each
  // wave builds Q~ = Q * s_tau for its tile's groups, hi and lo fp16 parts
  __shared__ uint32_t s_qb[KCH ? 4 : 1][KCH ? D / 2 : 1];
  constexpr int NGT = Stage<BITS, KCH, VCH, GRP>::NGT;
  __shared__ __align__(16) uint32_t s_qt[KCH ? kWaves : 1][KCH ? NGT : 1][2][4][KCH ? D / 2 + 4 : 4];
  float kq_sum[NGK];  // token-wise keys: sigma' * sum of head rh's query over each key group
  v8i qa[NQM];        // token-wise keys: query operand (rows 4 h + t, e4m3 terms t = 0, 1)
  int qsc[NQM];       // its E8M0 scale per row
  // query words, loaded before the first tiles are issued: the loads of one wave return in
  // issue order, so query loads behind a tile's would wait for the whole tile
  uint32_t qw[KCH ? 1 : 16];  // token-wise keys: the lane's 32 query values (MxKey::local order)
  uint32_t qgw[KCH ? 1 : 4];  // token-wise keys: head rh's channels 8 rq .. 8 rq + 7
  // rotated keys (ROT instances, rot bit 0): the query rows meet the keys as bf16(q H).  Wave w
  // loads row w (lane l: channels 2l, 2l + 1; channel-wise keys load it so anyway) and rotates it
  // once the first tiles are in flight; token-wise keys then take their operand words from the
  // rotated rows in LDS as they would from q.
  uint32_t qrow = 0u;
  auto query_load = [&]() {
   if (!KCH && ROT && (a.rot & 1)) {
    qrow = (wave < a.g_heads)
        ? reinterpret_cast<const uint32_t*>(a.q + ((size_t)b * a.hq + h * a.g_heads + wave) * D)[lane] : 0u;
    return;
   }
   if constexpr (KCH) {
    qw[0] = (wave < a.g_heads)
        ? reinterpret_cast<const uint32_t*>(a.q + ((size_t)b * a.hq + h * a.g_heads + wave) * D)[lane] : 0u;
   } else {
    const int hq = (lane & 15) >> 2, Gq = lane >> 4;
    const uint4* qr = reinterpret_cast<const uint4*>(
        a.q + ((size_t)b * a.hq + (size_t)h * a.g_heads + (hq < a.g_heads ? hq : 0)) * D);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = qr[MK::quad_index(Gq, i)];
      qw[4 * i] = u.x;
      qw[4 * i + 1] = u.y;
      qw[4 * i + 2] = u.z;
      qw[4 * i + 3] = u.w;
    }
    const uint32_t* qg = reinterpret_cast<const uint32_t*>(
        a.q + ((size_t)b * a.hq + (size_t)h * a.g_heads + (rh < a.g_heads ? rh : 0)) * D);
#pragma unroll
    for (int i = 0; i < 4; ++i) qgw[i] = qg[4 * rq + i];
   }
  };
  auto query_rotate = [&]() {  // (the query loads' wait falls after the first tiles' issue)
   if constexpr (ROT) {
    if (a.rot & 1) {
     if constexpr (KCH) {
      qw[0] = hadamard_bf16_pair(qw[0], lane);
     } else {
      __shared__ __align__(16) uint32_t s_qrot[kWaves][64];
      s_qrot[wave][lane] = hadamard_bf16_pair(qrow, lane);  // rows past G: zeros, never read
      __syncthreads();
      const int hq = (lane & 15) >> 2, Gq = lane >> 4;
      const uint4* qr = reinterpret_cast<const uint4*>(&s_qrot[hq < a.g_heads ? hq : 0][0]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 u = qr[MK::quad_index(Gq, i)];
        qw[4 * i] = u.x;
        qw[4 * i + 1] = u.y;
        qw[4 * i + 2] = u.z;
        qw[4 * i + 3] = u.w;
      }
      const uint32_t* qg = &s_qrot[rh < a.g_heads ? rh : 0][0];
#pragma unroll
      for (int i = 0; i < 4; ++i) qgw[i] = qg[4 * rq + i];
     }
    }
   }
  };
  auto query_prologue = [&]() {  // run after the first tiles are in flight, so the two HBM latencies overlap
   if constexpr (KCH) {
    if (wave < 4) s_qb[wave][lane] = qw[0];
    __syncthreads();
   } else {
    // A operand of the block-scaled QK^T: lane (G = lane / 16, row m = lane % 16), row
    // m = 4 h + (2 key group + term) (one key group: m = 4 h + t), bytes b = e4m3 term t of
    // query value (h, channel MK::chan(G, b)) masked to the row's key group, with one E8M0
    // scale per row from the row's largest value: two terms hold the 8 significant bits of
    // a bf16 value exactly
    {
      const int m = lane & 15, hq = m >> 2, slot = m & 3, Gq = lane >> 4;
      const bool hv = hq < a.g_heads;
      float qv[32];
#pragma unroll
      for (int bb = 0; bb < 32; ++bb) {
        const int l = MK::local(bb);
        const uint32_t w = qw[l >> 1];
        qv[bb] = __uint_as_float((l & 1) ? (w & 0xFFFF0000u) : (w << 16));
      }
#pragma unroll
      for (int r = 0; r < NQM; ++r) {
        const int jg = (NGK == 1) ? 0 : (NGK == 2) ? (slot >> 1) : 2 * r + (slot >> 1);
        const int t = (NGK == 1) ? slot : (slot & 1);
        const bool rv = hv && t < 2;
        float x[32], mx = 0.f;
#pragma unroll
        for (int bb = 0; bb < 32; ++bb) {
          x[bb] = (rv && MK::chan(Gq, bb) / GRP == jg) ? qv[bb] : 0.f;
          mx = fmaxf(mx, fabsf(x[bb]));
        }
        mx = max_halves(max_row_pairs(mx));  // the row's largest value over all 4 lane groups
        const int s0 = max((int)((__float_as_uint(mx) >> 23) & 0xFF) - 127, -100) - 7;  // largest in [128, 256)
        // e4m3 terms by the hardware conversions (OCP e4m3, round to nearest even, with
        // subnormals): term 0 of each value, and term 1 = 16 (value - term 0)
        v8i v;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x0 = __builtin_ldexpf(x[4 * i], -s0), x1 = __builtin_ldexpf(x[4 * i + 1], -s0);
          const float x2 = __builtin_ldexpf(x[4 * i + 2], -s0), x3 = __builtin_ldexpf(x[4 * i + 3], -s0);
          const int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false), true);
          const auto d01 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
          const auto d23 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
          const int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(
              (x2 - d23[0]) * 16.f, (x3 - d23[1]) * 16.f,
              __builtin_amdgcn_cvt_pk_fp8_f32((x0 - d01[0]) * 16.f, (x1 - d01[1]) * 16.f, 0, false), true);
          v[i] = (t == 1) ? w1 : w0;
        }
        qa[r] = v;
        qsc[r] = rv ? min(max(127 + s0 - 4 * t, 1), 254) : 127;
      }
    }
    // sigma' * sum of head rh's query over each key group: lane rq takes channels 8 rq .. 8 rq + 7
    {
      const bool hv = rh < a.g_heads;
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = hv ? qgw[i] : 0u;
        part += __uint_as_float(w << 16) + __uint_as_float(w & 0xFFFF0000u);
      }
#pragma unroll
      for (int jg = 0; jg < NGK; ++jg) kq_sum[jg] = row_sum16((8 * rq) / GRP == jg ? part : 0.f) * sl2;
    }
   }
  };
  // channel-wise K (operand-fold on Q): Q~ = Q * s_tau carried exactly as an fp16 pair hi + lo
  // (the fp32 product of a bf16 and an fp16 value is exact), and sigma' * (sum Q z - sum Q~ C)
  float kconst = 0.f;

  // ---- running state
  float m_ref = -INFINITY;                 // reference max of this lane's query (log2 units)
  float l_part = 0.f;                      // sum of p over this lane's quad tokens
  float vz_part[NGV], vb_part[NGV];        // token-wise V: sum p*(z + kMid s), sum P~ * (C + kMid) per value group
#pragma unroll
  for (int j = 0; j < NGV; ++j) vz_part[j] = vb_part[j] = 0.f;
  float ps_part = 0.f, pb_part = 0.f;      // channel-wise V: sum of P (fp32 if CENTER, else fp16), sum P16 * (C + kMid)
  f4 o_acc[2][2];                          // PV accumulators [channel 2l+h][quad parity]: rows = query heads
  f4 o_tot[2];                             // channel-wise V: folded output
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    o_acc[hh][0] = o_acc[hh][1] = f4{0.f, 0.f, 0.f, 0.f};
    o_tot[hh] = f4{0.f, 0.f, 0.f, 0.f};
  }
  uint32_t kc[C::NCONST];                  // operand-construction masks / exponents
#pragma unroll
  for (int i = 0; i < C::NCONST; ++i) kc[i] = in_vgpr(C::kConst[i]);

  // value-operand bias of this lane's quad (pairs 2*(qd % KPW), +1)
  const float cv0 = C::bias(2 * (pq % KPW)), cv1 = C::bias(2 * (pq % KPW) + 1);
  // rotated variant: value codes enter P V centred.  Each unit of P removes C + kMid (kMid = half
  // the code range, C + kMid exact in fp16) from the operand C + q, leaving q - kMid, and kMid * s *
  // (sum of the fp32 weights) joins the offset term.  The fp16 rounding errors of P then meet codes
  // of both signs instead of piling up in the same direction on every channel of a row, where the
  // rotation back by H would gather them into one channel.
  constexpr bool CENTER = ROT;
  constexpr float kMid = CENTER ? 0.5f * (float)((1 << BITS) - 1) : 0.f;
  const uint32_t cv0h = splat_f16(cv0 + kMid), cv1h = splat_f16(cv1 + kMid), oneh = splat_f16(1.f);

  const size_t bkv = bh / a.kv_group;  // the KV head this pair's query heads attend
  const uint32_t* kbase = a.pk + bkv * (size_t)a.tcap * KW;
  const uint32_t* vbase = a.pv + bkv * (size_t)(a.tcap / E) * D;
  const __amdgpu_buffer_rsrc_t rk = rsrc(kbase, (uint32_t)a.tcap * KW * 4);
  const __amdgpu_buffer_rsrc_t rv = rsrc(vbase, (uint32_t)(a.tcap / E) * D * 4);
  const uint16_t* ksb = a.ks + bkv * (size_t)(KCH ? (a.tcap / GRP) * D : a.tcap * NGK);
  const uint16_t* kzb = a.kz + bkv * (size_t)(KCH ? (a.tcap / GRP) * D : a.tcap * NGK);
  const uint16_t* vsb = a.vs + bkv * (size_t)(VCH ? (a.tcap / GRP) * D : a.tcap * NGV);
  const uint16_t* vzb = a.vz + bkv * (size_t)(VCH ? (a.tcap / GRP) * D : a.tcap * NGV);
  const uint32_t kscale_bytes = KCH ? (uint32_t)(a.tcap / GRP) * D * 2 : (uint32_t)a.tcap * NGK * 2;
  const uint32_t vscale_bytes = VCH ? (uint32_t)(a.tcap / GRP) * D * 2 : (uint32_t)a.tcap * NGV * 2;
  const __amdgpu_buffer_rsrc_t rks = rsrc(ksb, kscale_bytes);
  const __amdgpu_buffer_rsrc_t rkz = rsrc(kzb, kscale_bytes);
  const __amdgpu_buffer_rsrc_t rvs = rsrc(vsb, vscale_bytes);
  const __amdgpu_buffer_rsrc_t rvz = rsrc(vzb, vscale_bytes);
  // paged cache: lane l holds the pool block of the range's block blk0 + l (a range of at most
  // 63 blocks' tokens touches at most 64); a tile never crosses a block (blocks are whole tiles
  // and whole groups)
  const int P = PAGED ? a.block_size : 1;
  const int blk0 = PAGED ? r0 / P : 0;
  int blk_l = 0;
  if constexpr (PAGED) {
    const int nblk = (r1 - 1) / P - blk0 + 1;
    if (lane < nblk) blk_l = a.block_table[(size_t)b * (a.tcap / P) + blk0 + lane];
  }
  // one block's bytes of each array for one KV head
  const uint32_t kblk_bytes = (uint32_t)P * KW * 4, vblk_bytes = (uint32_t)(P / E) * D * 4;
  const uint32_t ksblk_bytes = KCH ? (uint32_t)(P / GRP) * D * 2 : (uint32_t)P * NGK * 2;
  const uint32_t vsblk_bytes = VCH ? (uint32_t)(P / GRP) * D * 2 : (uint32_t)P * NGV * 2;

  // rescale every accumulator of this wave after the reference max of a query moved
  auto rescale = [&](float alpha) {
    l_part *= alpha;
#pragma unroll
    for (int j = 0; j < NGV; ++j) {
      vz_part[j] *= alpha;
      vb_part[j] *= alpha;
    }
    ps_part *= alpha;
    pb_part *= alpha;
    float ai[4];
    if constexpr (KCH) {
      ai[0] = quad_bcast<0>(alpha); ai[1] = quad_bcast<1>(alpha); ai[2] = quad_bcast<2>(alpha); ai[3] = quad_bcast<3>(alpha);
    } else {  // head i's scores sit in row i
      ai[0] = lane_value(alpha, 0); ai[1] = lane_value(alpha, 16); ai[2] = lane_value(alpha, 32); ai[3] = lane_value(alpha, 48);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        o_acc[hh][0][i] *= ai[i];  // row i of the PV accumulators is query head i
        o_acc[hh][1][i] *= ai[i];
        o_tot[hh][i] *= ai[i];
      }
    }
  };

  // channel-wise V: fold the finished group tau into o_tot.  `span` = lanes whose quads form the group.
  auto fold_value_group = [&](uint32_t s2, uint32_t z2, int src_half) {
    // sums of the group per query, then broadcast query i's sums to every lane
    float psq[4], pbq[4];
    if constexpr (KCH) {
      float ps, pb;
      if (GRP == 32) {  // the group's quads are the lanes of half-wave src_half
        float a0, a1, b0, b1;
        halves(sum_same_query<32>(ps_part), a0, a1);
        halves(sum_same_query<32>(pb_part), b0, b1);
        ps = src_half ? a1 : a0;
        pb = src_half ? b1 : b0;
      } else {
        ps = sum_same_query<64>(ps_part);
        pb = sum_same_query<64>(pb_part);
      }
      psq[0] = quad_bcast<0>(ps); psq[1] = quad_bcast<1>(ps); psq[2] = quad_bcast<2>(ps); psq[3] = quad_bcast<3>(ps);
      pbq[0] = quad_bcast<0>(pb); pbq[1] = quad_bcast<1>(pb); pbq[2] = quad_bcast<2>(pb); pbq[3] = quad_bcast<3>(pb);
    } else {  // head i's quads are row i; a 32-token group is half a row (quads 0-7 or 8-15)
      const float ps = (GRP == 32) ? half_row_sum8(ps_part) : row_sum16(ps_part);
      const float pb = (GRP == 32) ? half_row_sum8(pb_part) : row_sum16(pb_part);
      const int o = (GRP == 32 && src_half) ? 8 : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        psq[i] = lane_value(ps, 16 * i + o);
        pbq[i] = lane_value(pb, 16 * i + o);
      }
    }
    const float sv[2] = {half_lo(s2), half_hi(s2)};
    const float zv[2] = {half_lo(z2), half_hi(z2)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        o_tot[hh][i] += sv[hh] * (o_acc[hh][0][i] + o_acc[hh][1][i]) +
                        ((CENTER ? fmaf(kMid, sv[hh], zv[hh]) : zv[hh]) * psq[i] - sv[hh] * pbq[i]);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) o_acc[hh][0] = o_acc[hh][1] = f4{0.f, 0.f, 0.f, 0.f};
  };

  // ---------------- tiles: staged in a per-wave LDS ring NS deep, read into registers
  struct Tile {
    uint4 k[KCH ? KW / 4 : 1];  // channel-wise keys: key row of token t0 + lane
    uint32_t kb[4][KCH ? 1 : MK::WPL];  // token-wise keys: packed words of block j's token 4 rq + j, lane group rh
    uint2 v[VW];               // value words of channels 2 lane, 2 lane + 1
    uint2 ks[NGK], kz[NGK];    // token-wise key (s, z) of the quad's tokens
    uint2 vs[NGV], vz[NGV];    // token-wise value (s, z) of the quad's tokens
    uint32_t kcs[NGT], kcz[NGT];  // channel-wise key (s, z) of channels 2 lane, 2 lane + 1, per group
    uint32_t vcs[NGT], vcz[NGT];  // channel-wise value (s, z), likewise
  };
  unsigned char* ring = smem + wave * NS * ST::BYTES;
  const uint32_t ring_lds = lds_addr(ring);
  // the wave's tiles in order: unit wave, wave + kWaves, ...; TPU tiles per unit
  auto tile_start = [&](int k) { return r0 + (wave + kWaves * (k / TPU)) * UNIT + (k % TPU) * kTile; };
  // tile at t0: HBM -> LDS slot k % NS (per-lane offsets fixed, tile offset scalar), from the
  // given buffer resources
  auto issue_from = [&](int k, uint32_t t0, const __amdgpu_buffer_rsrc_t& RK, const __amdgpu_buffer_rsrc_t& RV,
                        const __amdgpu_buffer_rsrc_t& RKS, const __amdgpu_buffer_rsrc_t& RKZ,
                        const __amdgpu_buffer_rsrc_t& RVS, const __amdgpu_buffer_rsrc_t& RVZ) {
    unsigned char* st = ring + (k % NS) * ST::BYTES;
    // scale blocks first, in layout order (see Stage), then K rows and V words
    if constexpr (!KCH) {
#pragma unroll
      for (int m = 0; m < ST::KSL; ++m) dma4(RKS, 4 * lane + 256 * m, t0 * NGK * 2, st + ST::SOFF + m * 256);
#pragma unroll
      for (int m = 0; m < ST::KSL; ++m) dma4(RKZ, 4 * lane + 256 * m, t0 * NGK * 2, st + ST::SOFF + ST::KSB + m * 256);
    }
    if constexpr (!VCH) {
#pragma unroll
      for (int m = 0; m < ST::VSL; ++m) dma4(RVS, 4 * lane + 256 * m, t0 * NGV * 2, st + ST::VSOFF + m * 256);
#pragma unroll
      for (int m = 0; m < ST::VSL; ++m) dma4(RVZ, 4 * lane + 256 * m, t0 * NGV * 2, st + ST::VSOFF + ST::VSB + m * 256);
    }
    if constexpr (KCH) {
#pragma unroll
      for (int g2 = 0; g2 < NGT; ++g2) dma4(RKS, 4 * lane, (t0 / GRP + g2) * D * 2, st + ST::KCOFF + g2 * 256);
#pragma unroll
      for (int g2 = 0; g2 < NGT; ++g2)
        dma4(RKZ, 4 * lane, (t0 / GRP + g2) * D * 2, st + ST::KCOFF + (NGT + g2) * 256);
    }
    if constexpr (VCH) {
#pragma unroll
      for (int g2 = 0; g2 < NGT; ++g2) dma4(RVS, 4 * lane, (t0 / GRP + g2) * D * 2, st + ST::VCOFF + g2 * 256);
#pragma unroll
      for (int g2 = 0; g2 < NGT; ++g2)
        dma4(RVZ, 4 * lane, (t0 / GRP + g2) * D * 2, st + ST::VCOFF + (NGT + g2) * 256);
    }
#pragma unroll
    for (int i = 0; i < KW / 4; ++i) dma16(RK, lane * KW * 4 + 16 * i, t0 * KW * 4, st + ST::KOFF + i * 1024);
#pragma unroll
    for (int i = 0; i < VW / 2; ++i) dma16(RV, 16 * lane + 1024 * i, (t0 / E) * D * 4, st + ST::VOFF + i * 1024);
  };
  // paged: the tile's block of the pool for this KV head (a block id outside the pool, or a tile
  // that is not there, gets resources of no bytes: out of range, no memory read, zeros)
  auto issue_paged = [&](int k, bool live) {
    const int t0 = tile_start(k);
    const int jj = live ? t0 / P - blk0 : 0;  // < 64: the host plans ranges of at most 63 blocks' tokens
    const int phys = (jj < 64) ? __builtin_amdgcn_readlane(blk_l, jj) : -1;
    const bool ok = live && phys >= 0 && phys < a.num_blocks;
    const size_t hb = ((size_t)(ok ? phys : 0) * (a.hkv / a.kv_group) + (size_t)h / a.kv_group);  // (block, head)
    const uint32_t tl0 = ok ? (uint32_t)(t0 % P) : 0u;
    issue_from(k, tl0, rsrc(a.pk + hb * ((size_t)P * KW), ok ? kblk_bytes : 0u),
               rsrc(a.pv + hb * ((size_t)(P / E) * D), ok ? vblk_bytes : 0u),
               rsrc(a.ks + hb * (ksblk_bytes / 2), ok ? ksblk_bytes : 0u), rsrc(a.kz + hb * (ksblk_bytes / 2), ok ? ksblk_bytes : 0u),
               rsrc(a.vs + hb * (vsblk_bytes / 2), ok ? vsblk_bytes : 0u), rsrc(a.vz + hb * (vsblk_bytes / 2), ok ? vsblk_bytes : 0u));
  };
  auto issue = [&](int k) {
    if constexpr (PAGED) issue_paged(k, true);
    else issue_from(k, (uint32_t)tile_start(k), rk, rv, rks, rkz, rvs, rvz);
  };
  // the first tiles: tile k, or (a wave with fewer) the same loads on resources of no bytes (out
  // of range: no memory read, zeros into a slot nobody reads).  The compiler counts loads to the
  // LDS in its waits only along straight-line code (at a join of branches holding such loads it
  // waits for all of them), and the query loads are waited for after these.
  auto issue_first = [&](int k, bool live) {
    if constexpr (PAGED) {
      issue_paged(k, live);
      return;
    }
    const uint32_t kb = live ? (uint32_t)a.tcap * KW * 4 : 0u, vb = live ? (uint32_t)(a.tcap / E) * D * 4 : 0u;
    const uint32_t ksz = live ? kscale_bytes : 0u, vsz = live ? vscale_bytes : 0u;  // scalar selects
    issue_from(k, live ? (uint32_t)tile_start(k) : 0u, rsrc(kbase, kb), rsrc(vbase, vb), rsrc(ksb, ksz),
               rsrc(kzb, ksz), rsrc(vsb, vsz), rsrc(vzb, vsz));
  };
  auto read = [&](Tile& tl, int k, int ahead) {  // wait for slot k % NS, LDS -> registers
    switch (ahead) {  // loads issued after this tile's that may still be in flight
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<ST::LOADS>(); break;
      case 2: wait_vmcnt<(NS > 2 ? 2 : 1) * ST::LOADS>(); break;
      default: wait_vmcnt<(NS - 1) * ST::LOADS>(); break;
    }
    const uint32_t st = ring_lds + (k % NS) * ST::BYTES;
    const uint32_t av = st + ST::VOFF + lane * 8;
    if constexpr (KCH) {
      const uint32_t ak = st + ST::KOFF + lane * 16;
      tl.k[0] = lds_b128<0>(ak);
      tl.k[1 % (KCH ? KW / 4 : 1)] = lds_b128<1024>(ak);
      if constexpr (KW / 4 > 2) {
        tl.k[2 % (KW / 4)] = lds_b128<2048>(ak);
        tl.k[3 % (KW / 4)] = lds_b128<3072>(ak);
      }
    } else {
      // key rows sit as 16-byte chunks [chunk][token]: lane group rh's codes of token 4 rq + j are
      // chunk rh / 2, bytes 8 (rh % 2) .. +7 (INT2), or chunk rh (INT4)
      if constexpr (BITS == 2) {
        const uint32_t ak = st + ST::KOFF + (rh >> 1) * 1024 + 64 * rq + 8 * (rh & 1);
        const uint2 w0 = lds_b64<0>(ak), w1 = lds_b64<16>(ak), w2 = lds_b64<32>(ak), w3 = lds_b64<48>(ak);
        tl.kb[0][0] = w0.x; tl.kb[0][1 % MK::WPL] = w0.y;
        tl.kb[1][0] = w1.x; tl.kb[1][1 % MK::WPL] = w1.y;
        tl.kb[2][0] = w2.x; tl.kb[2][1 % MK::WPL] = w2.y;
        tl.kb[3][0] = w3.x; tl.kb[3][1 % MK::WPL] = w3.y;
      } else {
        const uint32_t ak = st + ST::KOFF + rh * 1024 + 64 * rq;
        const uint4 w0 = lds_b128<0>(ak), w1 = lds_b128<16>(ak), w2 = lds_b128<32>(ak), w3 = lds_b128<48>(ak);
        const uint4 w[4] = {w0, w1, w2, w3};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          tl.kb[j][0] = w[j].x;
          tl.kb[j][1 % MK::WPL] = w[j].y;
          tl.kb[j][2 % MK::WPL] = w[j].z;
          tl.kb[j][3 % MK::WPL] = w[j].w;
        }
      }
    }
    tl.v[0] = lds_b64<0>(av);
    tl.v[1] = lds_b64<512>(av);
    tl.v[2] = lds_b64<1024>(av);
    tl.v[3] = lds_b64<1536>(av);
    if constexpr (VW > 4) {
      tl.v[4 % VW] = lds_b64<2048>(av);
      tl.v[5 % VW] = lds_b64<2560>(av);
      tl.v[6 % VW] = lds_b64<3072>(av);
      tl.v[7 % VW] = lds_b64<3584>(av);
    }
    if constexpr (!KCH) {
      const uint32_t as = st + ST::SOFF + pq * 8 * NGK;
      tl.ks[0] = lds_b64<0>(as);
      tl.kz[0] = lds_b64<ST::KSB>(as);
      if constexpr (NGK > 1) {
        tl.ks[1 % NGK] = lds_b64<8>(as);
        tl.kz[1 % NGK] = lds_b64<ST::KSB + 8>(as);
      }
      if constexpr (NGK > 2) {
        tl.ks[2 % NGK] = lds_b64<16>(as);
        tl.kz[2 % NGK] = lds_b64<ST::KSB + 16>(as);
        tl.ks[3 % NGK] = lds_b64<24>(as);
        tl.kz[3 % NGK] = lds_b64<ST::KSB + 24>(as);
      }
    }
    if constexpr (!VCH) {
      const uint32_t as = st + ST::VSOFF + pq * 8 * NGV;
      tl.vs[0] = lds_b64<0>(as);
      tl.vz[0] = lds_b64<ST::VSB>(as);
      if constexpr (NGV > 1) {
        tl.vs[1 % NGV] = lds_b64<8>(as);
        tl.vz[1 % NGV] = lds_b64<ST::VSB + 8>(as);
      }
      if constexpr (NGV > 2) {
        tl.vs[2 % NGV] = lds_b64<16>(as);
        tl.vz[2 % NGV] = lds_b64<ST::VSB + 16>(as);
        tl.vs[3 % NGV] = lds_b64<24>(as);
        tl.vz[3 % NGV] = lds_b64<ST::VSB + 24>(as);
      }
    }
    if constexpr (KCH) {
      const uint32_t ac = st + ST::KCOFF + lane * 4;
      tl.kcs[0] = lds_b32<0>(ac);
      tl.kcz[0] = lds_b32<NGT * 256>(ac);
      if constexpr (NGT > 1) {
        tl.kcs[1 % NGT] = lds_b32<256>(ac);
        tl.kcz[1 % NGT] = lds_b32<(NGT + 1) * 256>(ac);
      }
    }
    if constexpr (VCH) {
      const uint32_t ac = st + ST::VCOFF + lane * 4;
      tl.vcs[0] = lds_b32<0>(ac);
      tl.vcz[0] = lds_b32<NGT * 256>(ac);
      if constexpr (NGT > 1) {
        tl.vcs[1 % NGT] = lds_b32<256>(ac);
        tl.vcz[1 % NGT] = lds_b32<(NGT + 1) * 256>(ac);
      }
    }
    wait_lgkm0();
    if constexpr (KCH) {
#pragma unroll
      for (int i = 0; i < KW / 4; ++i) touch(tl.k[i]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int w = 0; w < MK::WPL; ++w) touch(tl.kb[j][w]);
    }
#pragma unroll
    for (int w = 0; w < VW; ++w) touch(tl.v[w]);
    if constexpr (!KCH) {
#pragma unroll
      for (int j = 0; j < NGK; ++j) { touch(tl.ks[j]); touch(tl.kz[j]); }
    }
    if constexpr (!VCH) {
#pragma unroll
      for (int j = 0; j < NGV; ++j) { touch(tl.vs[j]); touch(tl.vz[j]); }
    }
#pragma unroll
    for (int g2 = 0; g2 < NGT; ++g2) {
      if constexpr (KCH) { touch(tl.kcs[g2]); touch(tl.kcz[g2]); }
      if constexpr (VCH) { touch(tl.vcs[g2]); touch(tl.vcz[g2]); }
    }
  };

  auto process = [&](const Tile& tl, const int t0, auto tail_c) {
    constexpr bool tail = decltype(tail_c)::value;  // the tile reaches past T: mask its last tokens
    // ---------------- channel-wise K: the wave builds Q~ = Q * s_tau (hi, lo) for the tile's
    // groups in LDS, lane l taking channel pair l of every query head, and the score constant
    // sigma' * (sum_c Q z - sum_c Q~ C) of each (group, query head)
    if constexpr (KCH) {
      if (GRP <= kTile || t0 % GRP == 0) {
        const float cb = C::bias(lane % PAIRS);
        float kc[NGT];
#pragma unroll
        for (int g2 = 0; g2 < NGT; ++g2) {
          const uint32_t s2 = tl.kcs[g2], z2 = tl.kcz[g2];
          const float s0 = half_lo(s2), s1 = half_hi(s2), z0 = half_lo(z2), z1 = half_hi(z2);
          float part[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t w = s_qb[i][lane];
            const float q0 = __builtin_bit_cast(float, w << 16), q1 = __builtin_bit_cast(float, w & 0xFFFF0000u);
            const float pr0 = q0 * s0, pr1 = q1 * s1;  // exact
            const _Float16 h0 = (_Float16)pr0, h1 = (_Float16)pr1;
            const h2 hi = {h0, h1};
            const h2 lo = {(_Float16)(pr0 - (float)h0), (_Float16)(pr1 - (float)h1)};
            s_qt[wave][g2][0][i][lane] = as_u32(hi);
            s_qt[wave][g2][1][i][lane] = as_u32(lo);
            part[i] = fmaf(q0, z0, q1 * z1) - cb * (pr0 + pr1);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) part[i] = wave_sum(part[i]);
          kc[g2] = (qn == 0) ? part[0] : (qn == 1) ? part[1] : (qn == 2) ? part[2] : part[3];
        }
        kconst = ((NGT > 1 && qd >= 8) ? kc[NGT - 1] : kc[0]) * sl2;
        __builtin_amdgcn_wave_barrier();
      }
    }

    // ---------------- QK^T on the matrix cores
    float sc[4];
    if constexpr (!KCH) {
      // token-wise keys: block j (16 tokens, column n = token 4n + j) per block-scaled instruction,
      // key codes as fp4 / fp8 operands; lane 16 rh + rq receives head rh's raw scores of token
      // 4 rq + j in its rows (key group, term); the key-side fold (acc-fold: each group's partial
      // scaled once by s, plus z * sum(Q)) gives log2-unit scores before the softmax
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v8i bk = MK::build(tl.kb[j]);
        f4 c[NQM];
#pragma unroll
        for (int r = 0; r < NQM; ++r) c[r] = mx_mma<0, MK::FMT>(qa[r], bk, qsc[r], MK::CODE_SCALE);
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < NGK; ++q) {
          const int idx = j * NGK + q;  // fp16 index inside the quad's (token, group) block
          const uint2 sv = tl.ks[idx / 4];
          const uint2 zv = tl.kz[idx / 4];
          const uint32_t s32 = ((idx % 4) < 2) ? sv.x : sv.y;
          const uint32_t z32 = ((idx % 4) < 2) ? zv.x : zv.y;
          const float s = (idx % 2 == 0) ? half_lo(s32) : half_hi(s32);
          const float z = (idx % 2 == 0) ? half_lo(z32) : half_hi(z32);
          const f4& cq = c[(q / 2) % NQM];
          const float raw = (NGK == 1) ? cq[0] + cq[1] : cq[2 * (q % 2)] + cq[2 * (q % 2) + 1];
          acc = fmaf(s, raw * sl2, fmaf(z, kq_sum[q], acc));
        }
        sc[j] = acc;
        if (tail && (t0 + 4 * rq + j >= T)) sc[j] = -INFINITY;
      }
    } else {
      constexpr int NCH = 2;  // independent accumulation chains (hi and lo parts of Q~)
      f4 sacc[NCH];
  #pragma unroll
      for (int j = 0; j < NCH; ++j) sacc[j] = f4{0.f, 0.f, 0.f, 0.f};
      // B operand rows from LDS, re-read every tile (an opaque zero offset keeps
      // the compiler from hoisting them into 64 live registers)
      // One segment per key word (its KPW k-steps); the compiler may not move work
      // across segments, which bounds the live operands, and each segment reads
      // the next one's B operands from LDS ahead of use.
      // channel-wise K: hi parts (chain 0) and lo parts (chain 1) of Q~ for this lane's group
      const int opq = (int)in_vgpr(0u);
      const int g2l = (KCH && NGT > 1 && qd >= 8) ? 1 : 0;
      const uint4* qsrc = reinterpret_cast<const uint4*>(&s_qt[KCH ? wave : 0][g2l][0][qn][0]) + opq;
      const uint4* qlsrc = reinterpret_cast<const uint4*>(&s_qt[KCH ? wave : 0][g2l][1][qn][0]) + opq;
      uint4 qcur[QPW], qnxt[QPW], lcur[KCH ? QPW : 1], lnxt[KCH ? QPW : 1];
  #pragma unroll
      for (int i = 0; i < QPW; ++i) qcur[i] = qsrc[i];
      if constexpr (KCH) {
  #pragma unroll
        for (int i = 0; i < QPW; ++i) lcur[i] = qlsrc[i];
      }
      uint4 kseg;
  #pragma unroll
      for (int d = 0; d < KW; ++d) {
        if (d % 4 == 0) kseg = tl.k[d / 4];
        if (d + 1 < KW) {
  #pragma unroll
          for (int i = 0; i < QPW; ++i) qnxt[i] = qsrc[(d + 1) * QPW + i];
          if constexpr (KCH) {
  #pragma unroll
            for (int i = 0; i < QPW; ++i) lnxt[i] = qlsrc[(d + 1) * QPW + i];
          }
        }
        if (d % 4 == 0) touch(kseg);  // ties the unpacking of these four words to this segment onwards
        const uint32_t wrd = (d % 4 == 0) ? kseg.x : (d % 4 == 1) ? kseg.y : (d % 4 == 2) ? kseg.z : kseg.w;
        uint32_t p[PAIRS];
        C::extract(wrd, kc, p);
  #pragma unroll
        for (int sg = 0; sg < KPW; ++sg) {
          const int j = d * KPW + sg;  // k-step: channels 4j .. 4j+3
          const h4 av = cat4(p[2 * sg], p[2 * sg + 1]);
          (void)j;
          const uint4 qh = qcur[sg / 2], ql = lcur[sg / 2];
          const h4 bh = (sg & 1) ? cat4(qh.z, qh.w) : cat4(qh.x, qh.y);
          const h4 bl = (sg & 1) ? cat4(ql.z, ql.w) : cat4(ql.x, ql.y);
          sacc[0] = __builtin_amdgcn_mfma_f32_4x4x4f16(av, bh, sacc[0], 0, 0, 0);
          sacc[1] = __builtin_amdgcn_mfma_f32_4x4x4f16(av, bl, sacc[1], 0, 0, 0);
        }
  #pragma unroll
        for (int i = 0; i < QPW; ++i) qcur[i] = qnxt[i];
        if constexpr (KCH) {
  #pragma unroll
          for (int i = 0; i < QPW; ++i) lcur[i] = lnxt[i];
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---------------- key-side fold (before the softmax) -> scores in log2 units
  #pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[r] = fmaf(sacc[0][r] + sacc[1][r], sl2, kconst);
        if (tail && (t0 + 4 * qd + r >= T)) sc[r] = -INFINITY;
      }
    }

    // ---------------- online softmax: exact running max per query head.  The
    // largest weight seen so far is exactly 1, so the operand-folded weight of
    // the dominant token (p * s) is its fp16 scale itself, with no rounding.
    const float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    const float m_new = KCH ? wave_max_same_query_and(mt, m_ref) : row_max16_and(mt, m_ref);
    if (__any(m_new > m_ref)) {
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);  // 0 on the first tile
      m_ref = m_new;
      rescale(alpha);
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sc[r] - m_ref);
    l_part += (p[0] + p[1]) + (p[2] + p[3]);

    // ---------------- P operands (value-side operand-fold for token-wise V)
    if constexpr (!VCH) {
#pragma unroll
      for (int j = 0; j < NGV; ++j) {
        float s[4], z[4];
        uint32_t sw[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int idx = r * NGV + j;
          const uint2 sv = tl.vs[idx / 4];
          const uint2 zv = tl.vz[idx / 4];
          const uint32_t s32 = ((idx % 4) < 2) ? sv.x : sv.y;
          const uint32_t z32 = ((idx % 4) < 2) ? zv.x : zv.y;
          sw[r] = s32;
          s[r] = (idx % 2 == 0) ? half_lo(s32) : half_hi(s32);
          z[r] = (idx % 2 == 0) ? half_lo(z32) : half_hi(z32);
          if (tail && (t0 + 4 * pq + r >= T)) s[r] = z[r] = 0.f;  // padding may hold NaN
          if constexpr (CENTER) z[r] = fmaf(kMid, s[r], z[r]);  // offset of the centred codes
        }
        uint32_t p01, p23;
        if constexpr (tail) {
          p01 = pack_f16(p[0] * s[0], p[1] * s[1]);
          p23 = pack_f16(p[2] * s[2], p[3] * s[3]);
        } else {  // straight from the fp16 scales, one rounding per product
          p01 = mul_f16x2(p[0], sw[0], (0 * NGV + j) % 2, p[1], sw[1], (1 * NGV + j) % 2);
          p23 = mul_f16x2(p[2], sw[2], (2 * NGV + j) % 2, p[3], sw[3], (3 * NGV + j) % 2);
        }
        s_p[wave][j][KCH ? qn : rh][pq] = make_uint2(p01, p23);
        vb_part[j] = dot2(p23, cv1h, dot2(p01, cv0h, vb_part[j]));
        vz_part[j] = fmaf(p[0], z[0], fmaf(p[1], z[1], fmaf(p[2], z[2], fmaf(p[3], z[3], vz_part[j]))));
      }
    } else {
      const uint32_t p01 = pack_f16(p[0], p[1]);
      const uint32_t p23 = pack_f16(p[2], p[3]);
      s_p[wave][0][KCH ? qn : rh][pq] = make_uint2(p01, p23);
      if constexpr (CENTER)
        ps_part += (p[0] + p[1]) + (p[2] + p[3]);  // fp32 weights
      else
        ps_part = dot2(p23, oneh, dot2(p01, oneh, ps_part));
      pb_part = dot2(p23, cv1h, dot2(p01, cv0h, pb_part));
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // A operands: P of query qn for the 16 quads (value group of this lane's
    // channels), gathered from LDS one segment ahead of use
    const int jv = VCH ? 0 : (8 * qd) / GRP;
    const uint4* psrc = reinterpret_cast<const uint4*>(&s_p[wave][jv][qn][0]);
    uint4 pcur[QPW], pnxt[QPW];
#pragma unroll
    for (int i = 0; i < QPW; ++i) pcur[i] = psrc[i];

    // ---------------- P V on the matrix cores (+ acc-fold of channel-wise value groups)
#pragma unroll
    for (int w = 0; w < VW; ++w) {
      if (w + 1 < VW) {
#pragma unroll
        for (int i = 0; i < QPW; ++i) pnxt[i] = psrc[(w + 1) * QPW + i];
      }
      uint2 vw = tl.v[w];
      touch(vw);  // ties the unpacking to this segment
      const uint32_t vx = vw.x, vy = vw.y;
      uint32_t p0[PAIRS], p1[PAIRS];
      C::extract(vx, kc, p0);  // channel 2*lane
      C::extract(vy, kc, p1);  // channel 2*lane + 1
#pragma unroll
      for (int sg = 0; sg < KPW; ++sg) {
        const int bq = w * KPW + sg;  // quad: tokens 4bq .. 4bq+3 of the tile
        const uint4 pp = pcur[sg / 2];
        const h4 av = (sg & 1) ? cat4(pp.z, pp.w) : cat4(pp.x, pp.y);
        f4& a0 = o_acc[0][bq & 1];
        f4& a1 = o_acc[1][bq & 1];
        a0 = __builtin_amdgcn_mfma_f32_4x4x4f16(av, cat4(p0[2 * sg], p0[2 * sg + 1]), a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_4x4x4f16(av, cat4(p1[2 * sg], p1[2 * sg + 1]), a1, 0, 0, 0);
        if constexpr (VCH && GRP == 32) {
          if (bq == 7) {  // first 32-token group of the tile is complete
            if (t0 < T) fold_value_group(tl.vcs[0], tl.vcz[0], 0);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < QPW; ++i) pcur[i] = pnxt[i];
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_wave_barrier();
    if constexpr (VCH) {
      if (GRP == 32) {
        if (t0 + 32 < T) fold_value_group(tl.vcs[NGT - 1], tl.vcz[NGT - 1], 1);
        else {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) o_acc[hh][0] = o_acc[hh][1] = f4{0.f, 0.f, 0.f, 0.f};
        }
        ps_part = pb_part = 0.f;
      } else if ((t0 + kTile) % GRP == 0 || t0 + kTile >= r1) {
        fold_value_group(tl.vcs[0], tl.vcz[0], 0);
        ps_part = pb_part = 0.f;
      }
    }
  };

  int nt = 0;  // tiles of this wave
  while (tile_start(nt) < r1) ++nt;
  // The SIMD issues from the oldest ready wave first, so the work-groups
  // dispatched first would race ahead and the last ones would finish alone.
  // Each wave lowers its priority at every quarter of its tiles: waves that
  // are behind win the arbitration and all of them finish together.  The
  // prologue runs at the top priority: at the default one, a wave still
  // building its query operand waited behind the loops of the waves around it.
  const int q1 = nt / 4, q2 = nt / 2, q3 = (3 * nt) / 4;
  __builtin_amdgcn_s_setprio(3);
  query_load();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < NS; ++k) issue_first(k, k < nt);
  query_rotate();
  query_prologue();
  timeline_mark(1);
  // Tiles start in increasing order and stop below T, so only the wave's last
  // tile can reach past T.  It is peeled off the loop: a loop body with one
  // instance of the tile code keeps its accumulators in the same registers
  // from one iteration to the next (two instances merging in the loop made
  // the compiler copy them back at every iteration).
  for (int k = 0; k < nt - 1; ++k) {
    if (k == q1) __builtin_amdgcn_s_setprio(2);
    if (k == q2) __builtin_amdgcn_s_setprio(1);
    if (k == q3) __builtin_amdgcn_s_setprio(0);
    Tile tl;
    read(tl, k, min(NS - 1, nt - 1 - k));
    if (k + NS < nt) issue(k + NS);  // the slot just read: NS tiles in flight while this one is processed
    process(tl, tile_start(k), std::false_type{});
  }
  if (nt > 0) {
    __builtin_amdgcn_s_setprio(0);  // q3 <= nt - 1: the last tile always ran at the lowest priority
    Tile tl;
    read(tl, nt - 1, 0);  // (and any loads on no bytes: done before the rings are reused)
    const int t0k = tile_start(nt - 1);
    if (t0k + kTile > T)
      process(tl, t0k, std::true_type{});
    else
      process(tl, t0k, std::false_type{});
  } else {
    wait_vmcnt<0>();  // the loads on no bytes write the ring: done before it is reused
  }

  timeline_mark(2);
  __builtin_amdgcn_s_setprio(3);  // the epilogue and the merge are the tail of the launch
  // persistent work-groups: the next item's index and lengths load during the epilogue
  NextLoad nx;
  if (next && wave == 0) next_load(a, nx);

  // ---------------- wave epilogue: totals per query, value-side corrections
  // (channel-wise keys: a query head's lanes are those of one l & 3; token-wise keys: one row)
  const float l_tot = KCH ? sum_same_query<64>(l_part) : row_sum16(l_part);
  f4 o_fin[2];
  if constexpr (VCH) {
    o_fin[0] = o_tot[0];
    o_fin[1] = o_tot[1];
  } else {
    const int jv = (8 * qd) / GRP;  // value group of channels 2l, 2l+1
    float cq[4];  // correction of this lane's value group for query head i
    if constexpr (KCH) {
      float zc[NGV], bc[NGV];
#pragma unroll
      for (int j = 0; j < NGV; ++j) {
        zc[j] = sum_same_query<64>(vz_part[j]);
        bc[j] = sum_same_query<64>(vb_part[j]);
      }
      float cg = 0.f;  // correction of this lane's value group, per this lane's query head
#pragma unroll
      for (int j = 0; j < NGV; ++j) cg = (j == jv) ? zc[j] - bc[j] : cg;
      cq[0] = quad_bcast<0>(cg); cq[1] = quad_bcast<1>(cg); cq[2] = quad_bcast<2>(cg); cq[3] = quad_bcast<3>(cg);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) cq[i] = 0.f;
#pragma unroll
      for (int j = 0; j < NGV; ++j) {
        const float dj = row_sum16(vz_part[j]) - row_sum16(vb_part[j]);  // head rh's correction of group j
#pragma unroll
        for (int i = 0; i < 4; ++i) cq[i] = (j == jv) ? lane_value(dj, 16 * i) : cq[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float corr = cq[i];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) o_fin[hh][i] = (o_acc[hh][0][i] + o_acc[hh][1][i]) + corr;
    }
  }
  __syncthreads();  // every wave is done with its ring before the rings hold s_o
  if (KCH ? lane < 4 : rq == 0) {  // one lane per query head
    s_ml[wave][0][KCH ? lane : rh] = m_ref;
    s_ml[wave][1][KCH ? lane : rh] = l_tot;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s_o[wave][i][2 * lane] = o_fin[0][i];
    s_o[wave][i][2 * lane + 1] = o_fin[1][i];
  }
  __syncthreads();

  finish_range<UNIT, ROT>(a, b, h, split, T, s_ml, s_o, next, nx);
}

// A full-precision window of recent tokens attended by S more work-groups of
// the pair (grid rows 0 .. S-1, dispatched first, work-group j taking window
// tokens [j * chunk, +chunk)), concurrently with the pair's cache ranges (the
// rows after them; the plan leaves S slots per pair for them):
// the window's keys and values are further tokens of the same softmax.  The
// work-group writes its normalised partial and lse to its window slot with
// device-coherent stores and arrives at the pair's counter like a range; the
// last arrival merges (merge_ranges folds the slots in).  A sequence with no
// cache token and a single window work-group takes that partial as output.
// Scores come from bf16 x bf16 products in fp32.  LDS: the query rows, the
// score table and the waves' partial sums reuse the tile rings.
__device__ __forceinline__ float wg_reduce(float v, float* red, bool is_max) {
  for (int m = 32; m >= 1; m >>= 1) {
    const float o = __shfl_xor(v, m);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  __syncthreads();  // red is free
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

template <bool ROT>
__device__ __forceinline__ void window_item(const SplitArgs& a, const int b, const int h, const int T, const int j) {
  constexpr int D = kHeadDim;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float s_wred[kWaves];
  const int CW = a.win_chunk;                    // window tokens of one work-group
  float* s_p = reinterpret_cast<float*>(smem) + kMaxG * D;  // [kMaxG][CW] (after a [kMaxG][D] area left free)
  float* s_ow = s_p + kMaxG * CW;                // [kWaves][kMaxG][D]
  const int G = a.g_heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.win_wgs;
  // this work-group's window tokens: [j * CW, j * CW + W)
  const int W = min(max(min(max(a.win_lens[b], 0), a.win_cap) - j * CW, 0), CW);
  const int chunk = (W + kWaves - 1) / kWaves;
  const int t0 = wave * chunk, t1 = min(t0 + chunk, W);
  const size_t row0 = (size_t)b * a.hq + (size_t)h * G;
  const size_t bh = (size_t)b * a.hkv + h;
  const size_t kv0 = ((bh / a.kv_group) * (size_t)a.win_cap + (size_t)j * CW) * D;  // the pair's KV head
  // scores on the matrix cores: v_mfma_f32_16x16x32_bf16 with A = 16 window keys (rows = tokens),
  // B = the query rows (columns; G of 16 used), the contraction over channels in 4 steps of 32.
  // Lane l holds token / query row l % 16 and, at step k, channels 32k + 8(l / 16) .. +7 of both
  // operands (A and B take the same slot layout, so any assignment of channels to slots that both
  // share gives the full dot product).  bf16 x bf16 products are exact in fp32.  C: lane l holds
  // tokens 4(l / 16) .. +3 of the block for query row l % 16.
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int mr = lane & 15, mg = lane >> 4;
  bf16x8 qb[D / 32];
  {
    const uint32_t* qr = reinterpret_cast<const uint32_t*>(a.q + (row0 + (size_t)min(mr, G - 1)) * D);
#pragma unroll
    for (int k = 0; k < D / 32; ++k) {
      uint4 w;  // 4-byte loads: the query is only 4-byte aligned
      w.x = qr[(32 * k + 8 * mg) / 2 + 0];
      w.y = qr[(32 * k + 8 * mg) / 2 + 1];
      w.z = qr[(32 * k + 8 * mg) / 2 + 2];
      w.w = qr[(32 * k + 8 * mg) / 2 + 3];
      if (mr >= G) w = make_uint4(0u, 0u, 0u, 0u);
      qb[k] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const uint4* wk = reinterpret_cast<const uint4*>(a.win_k + kv0);
  // key rows of block tb (rows past t1 re-read row t1 - 1); the next block's rows load while this
  // block's scores are formed, so a wave keeps two blocks in flight instead of one
  auto load_keys = [&](uint4 (&kw)[D / 32], int tb) {
    const uint4* kr = wk + (size_t)min(tb + mr, t1 - 1) * (D / 8) + mg;
#pragma unroll
    for (int k = 0; k < D / 32; ++k) kw[k] = kr[4 * k];
  };
  uint4 kw[D / 32], kn[D / 32] = {};
  if (t0 < t1) load_keys(kw, t0);
  for (int tb = t0; tb < t1; tb += 16) {  // wave-uniform: the matrix instructions run with every lane
    if (tb + 16 < t1) load_keys(kn, tb + 16);
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < D / 32; ++k)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw[k]), qb[k], c, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = tb + 4 * mg + r;
      if (mr < G && tr < t1) s_p[mr * CW + tr] = c[r] * a.win_sm;
    }
#pragma unroll
    for (int k = 0; k < D / 32; ++k) kw[k] = kn[k];
  }
  __syncthreads();
  float m[kMaxG], l[kMaxG];
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    float v = -INFINITY;
    for (int t = tid; t < W; t += kWaves * 64) v = fmaxf(v, s_p[i * CW + t]);
    m[i] = wg_reduce(v, s_wred, true);
    float sum = 0.f;
    for (int t = tid; t < W; t += kWaves * 64) {
      const float p = __expf(s_p[i * CW + t] - m[i]);
      s_p[i * CW + t] = p;
      sum += p;
    }
    l[i] = wg_reduce(sum, s_wred, false);
  }
  __syncthreads();
  const uint32_t* wv = reinterpret_cast<const uint32_t*>(a.win_v + kv0) + lane;
  float o[kMaxG][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
  // value rows of tokens tb .. tb + 15 (zeros past t1), one block ahead as for the keys
  auto load_values = [&](uint32_t (&vr)[16], int tb) {
#pragma unroll
    for (int u = 0; u < 16; ++u) vr[u] = (tb + u < t1) ? wv[(size_t)(tb + u) * (D / 2)] : 0u;
  };
  uint32_t vr[16], vn[16] = {};
  if (t0 < t1) load_values(vr, t0);
  for (int tb = t0; tb < t1; tb += 16) {
    if (tb + 16 < t1) load_values(vn, tb + 16);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (tb + u >= t1) break;
      const float v0 = __uint_as_float(vr[u] << 16), v1 = __uint_as_float(vr[u] & 0xFFFF0000u);
#pragma unroll
      for (int i = 0; i < kMaxG; ++i) {
        const float p = s_p[i * CW + tb + u];
        o[i][0] = fmaf(p, v0, o[i][0]);
        o[i][1] = fmaf(p, v1, o[i][1]);
      }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) vr[u] = vn[u];
  }
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    s_ow[(wave * kMaxG + i) * D + 2 * lane] = o[i][0];
    s_ow[(wave * kMaxG + i) * D + 2 * lane + 1] = o[i][1];
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kWaves * 64) {
    const int i = idx / D, c = idx % D;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += s_ow[(w * kMaxG + i) * D + c];
    const float li = (i == 0) ? l[0] : (i == 1) ? l[1] : (i == 2) ? l[2] : l[3];
    const float mi = (i == 0) ? m[0] : (i == 1) ? m[1] : (i == 2) ? m[2] : m[3];
    const float ow = (W == 0) ? 0.f : sum / li, lw = (W == 0) ? -INFINITY : mi + __logf(li);
    const size_t row = row0 + i;
    if (T == 0 && S == 1) {  // no cache range and one window partial: it is the output
      a.out[row * D + c] = to_bf16_rne(ow);
      if (c == 0 && a.lse) a.lse[row] = lw;
    } else {
      __hip_atomic_store(a.win_o + (row * S + j) * D + c, ow, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (c == 0) __hip_atomic_store(a.win_lse + row * S + j, lw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (T == 0 && S == 1) return;
  const int ns = (T + a.chunk - 1) / a.chunk;
  __shared__ int s_wlast;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int done = __hip_atomic_fetch_add(a.counters + bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_wlast = (done == ns + S - 1);  // ns ranges and S window work-groups arrive
  }
  __syncthreads();
  if (!s_wlast) return;
  merge_ranges<ROT>(a, b, h, ns);
  if (tid == 0) a.counters[bh] = 0;
}

// Grids that fit the device in one round: the grid's own map (work-group
// (x, y): window row y of pair x, or range y of pair (x + y) mod pairs).
// Larger grids (ragged batches of at most kMapMaxB sequences) run persistent:
// one round of work-groups takes work items from a device-wide counter, longest
// first (map_select), until the items run out; the last work-group to leave
// resets the counters for the next call.  A window's work-groups come before
// that round in the grid, one item each; no work-group ever waits for another
// (every hand-off is an arrival count), so their order cannot stall the grid.
template <int BITS, bool KCH, bool VCH, int GRP, bool PAGED, bool ROT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(waves_per_simd<BITS, KCH, VCH, GRP>())))
void split_decode(const SplitArgs a) {
  if (!a.persistent) {
    // Work-group (x, y) runs pair x's window row y (y < win_wgs), or range
    // y - win_wgs of pair (x + y) mod B*Hkv: work-groups are dealt to the XCDs
    // round-robin in launch order, and the rotation spreads each pair's ranges
    // over all of them (without it, every range of pair x ran on XCD x % 8).
    const bool win = (int)blockIdx.y < a.win_wgs;
    const int pair = win ? (int)blockIdx.x : ((int)blockIdx.x + (int)blockIdx.y) % (int)gridDim.x;
    const int b = pair / a.hkv;
    const int T = min(max(a.seq_lens[b], 0), a.tcap);
    if (win) {  // dispatched first: run beside the ranges, not after them
      window_item<ROT>(a, b, pair % a.hkv, T, blockIdx.y);
      return;
    }
    timeline_item(0);
    timeline_mark(0);
    timeline_hw();
    timeline_set(5, (unsigned long long)b << 40 | (unsigned long long)pair << 20 | (blockIdx.y - a.win_wgs));
    run_item<BITS, KCH, VCH, GRP, PAGED, ROT>(a, b, pair % a.hkv, (int)blockIdx.y - a.win_wgs, T, nullptr);
    timeline_mark(4);
    return;
  }
  // window work-groups take the first blocks (dispatched first) and leave
  // after their one item; they never take an item from the counter
  const int pairs = a.batch * a.hkv;
  const int nwin = pairs * a.win_wgs;
  if ((int)blockIdx.x < nwin) {
    const int pair = (int)blockIdx.x % pairs;  // consecutive blocks: different pairs
    const int b = pair / a.hkv;
    window_item<ROT>(a, b, pair % a.hkv, min(max(a.seq_lens[b], 0), a.tcap), (int)blockIdx.x / pairs);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  __shared__ int s_item[5];  // the next item: {b, h, range, kind, T}
  if (wave == 0) {
    NextLoad nx;
    next_load(a, nx);
    map_select<work_unit<KCH, VCH, GRP>()>(a, nx, s_item);
  }
  __syncthreads();
  int item_no = 0;  // (the timeline's item number)
  for (;;) {
    const int kind = __builtin_amdgcn_readfirstlane(s_item[3]);
    const int b = __builtin_amdgcn_readfirstlane(s_item[0]);
    const int h = __builtin_amdgcn_readfirstlane(s_item[1]);
    const int split = __builtin_amdgcn_readfirstlane(s_item[2]);
    const int T = __builtin_amdgcn_readfirstlane(s_item[4]);
    __syncthreads();  // s_item is read before wave 0 maps the item after this one into it
    if (kind == kItemNone) break;
    timeline_item(item_no++);
    timeline_mark(0);
    timeline_hw();
    timeline_set(5, (unsigned long long)b << 40 | (unsigned long long)(b * a.hkv + h) << 20 | (unsigned)split);
    run_item<BITS, KCH, VCH, GRP, PAGED, ROT>(a, b, h, split, T, s_item);
    timeline_mark(4);
    __syncthreads();  // the item's LDS is free and s_item holds the next item
  }
  if (threadIdx.x == 0) {
    const int left = __hip_atomic_fetch_add(a.work_ctr + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (left == (int)gridDim.x - nwin - 1) {  // every other item-taking work-group has left: no more grabs
      __hip_atomic_store(a.work_ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.work_ctr + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Launch the instantiation on `stream`, or (per_cu != nullptr) report how many
// of its work-groups one CU holds at once instead.
template <int BITS, bool KCH, bool VCH, int GRP, bool PAGED, bool ROT>
hipError_t launch_one(int batch, int hkv, const SplitArgs& sa, hipStream_t stream, int* per_cu, const LaunchEvents& ev) {
  using ST = Stage<BITS, KCH, VCH, GRP>;
  constexpr size_t lds = (size_t)kWaves * ST::NS * ST::BYTES;
  static_assert(lds >= sizeof(float) * kWaves * 4 * kHeadDim, "rings must hold the epilogue buffer");
  // the work-group's LDS (static + rings) must fit one CU, or the dispatch
  // would be rejected on the device and abort the queue: refuse it here
  static int lds_ok = -1;  // per instantiation: -1 unknown, 0 too big, 1 fits
  if (lds_ok < 0) {
    hipFuncAttributes fa;
    int dev = 0, cu_lds = 0;
    if (hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(split_decode<BITS, KCH, VCH, GRP, PAGED, ROT>)) != hipSuccess ||
        hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cu_lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess)
      return hipErrorInvalidDeviceFunction;
    lds_ok = (fa.sharedSizeBytes + lds <= (size_t)cu_lds) ? 1 : 0;
  }
  if (!lds_ok) return hipErrorInvalidConfiguration;
  if (per_cu)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, split_decode<BITS, KCH, VCH, GRP, PAGED, ROT>, kWaves * 64, lds);
  static_assert(lds >= sizeof(float) * (kMaxG * kHeadDim * (1 + kWaves) + kMaxG * kFusedWindowMax),
                "rings must hold a fused window's query rows, scores and partial sums");
  const dim3 grid = sa.persistent ? dim3(sa.grid_wgs + batch * hkv * sa.win_wgs) : dim3(batch * hkv, sa.splits + sa.win_wgs);
  if (ev.start || ev.stop)  // timing events recorded by the dispatch itself
    hipExtLaunchKernelGGL((split_decode<BITS, KCH, VCH, GRP, PAGED, ROT>), grid, dim3(kWaves * 64), lds, stream, ev.start, ev.stop,
                          0, sa);
  else
    hipLaunchKernelGGL((split_decode<BITS, KCH, VCH, GRP, PAGED, ROT>), grid, dim3(kWaves * 64), lds, stream, sa);
  return hipGetLastError();
}

template <int BITS, bool KCH, bool VCH, bool PAGED, bool ROT>
hipError_t launch_gp(int group, int batch, int hkv, const SplitArgs& sa, hipStream_t stream, int* per_cu,
                     const LaunchEvents& ev) {
  switch (group) {
    case 32: return launch_one<BITS, KCH, VCH, 32, PAGED, ROT>(batch, hkv, sa, stream, per_cu, ev);
    case 64: return launch_one<BITS, KCH, VCH, 64, PAGED, ROT>(batch, hkv, sa, stream, per_cu, ev);
    case 128: return launch_one<BITS, KCH, VCH, 128, PAGED, ROT>(batch, hkv, sa, stream, per_cu, ev);
  }
  return hipErrorInvalidValue;
}

// Every (bits, layout, group) instance of one (paged, rotated) variant: launch, or with per_cu
// set, report its occupancy instead.  Each variant is instantiated in a source file of its own.
template <bool PAGED, bool ROT>
hipError_t launch_variant(int bits, bool kch, bool vch, int group, int batch, int hkv, const SplitArgs& sa,
                          hipStream_t stream, int* per_cu, const LaunchEvents& ev) {
  if (bits == 2) {
    if (kch) return vch ? launch_gp<2, true, true, PAGED, ROT>(group, batch, hkv, sa, stream, per_cu, ev)
                        : launch_gp<2, true, false, PAGED, ROT>(group, batch, hkv, sa, stream, per_cu, ev);
    return vch ? launch_gp<2, false, true, PAGED, ROT>(group, batch, hkv, sa, stream, per_cu, ev)
               : launch_gp<2, false, false, PAGED, ROT>(group, batch, hkv, sa, stream, per_cu, ev);
  }
  if (kch) return vch ? launch_gp<4, true, true, PAGED, ROT>(group, batch, hkv, sa, stream, per_cu, ev)
                      : launch_gp<4, true, false, PAGED, ROT>(group, batch, hkv, sa, stream, per_cu, ev);
  return vch ? launch_gp<4, false, true, PAGED, ROT>(group, batch, hkv, sa, stream, per_cu, ev)
             : launch_gp<4, false, false, PAGED, ROT>(group, batch, hkv, sa, stream, per_cu, ev);
}
}  // namespace
}  // namespace foscar
