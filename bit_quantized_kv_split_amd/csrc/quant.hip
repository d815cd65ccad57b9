// Quantise-and-append: new keys and values (bf16) into the packed 2-/4-bit
// cache that the decode kernel reads, gfx950.
//
// Encoding: value = s*q + z with one scale s and one offset z per group of
// codes ("FOSCAR speeds up 2-bit KV decode -- Affine folding of KV
// dequantization", learnaivisually, encoding paragraph); a group runs along
// the channels of one token (token-wise) or along the tokens of one channel
// (channel-wise), the fold-placement table of the same page.  The pages give
// no quantiser; this is min-max asymmetric quantisation with its decisions in
// fp32: s = fp16((max - min) / (2^bits - 1)), z = fp16(min),
// q = rint((x - z) / s) clamped to the code range (q = 0 when s = 0).
//
// Work decomposition: one wave per (128-token block, KV head, sequence),
// stepping four tokens at a time.  Lane l takes token slot l / 16 of the step
// and channels 8 (l % 16) .. +7: one 16-byte load per lane, four consecutive
// 256-byte rows per wave-instruction.
//   * token-wise group (g channels of a token = g/8 lanes of one slot):
//     min / max inside the lane, then DPP quad swaps and row mirrors;
//   * channel-wise group (g tokens of a channel): each lane folds its slot's
//     tokens of the group into min / max of its 8 channels, the four slots are
//     combined by permlane swaps, then the group's rows are read again (from
//     L2) to code them;
//   * codes: rint((x - z) * rcp(s)); a lane whose product lies within 2^-16 of
//     a half-integer takes the correctly rounded division instead, so every
//     code equals rint of the fp32 quotient;
//   * keys are packed along channels: a lane's 8 codes fill half an INT2 word
//     (one DPP OR with the neighbour octet) or a whole INT4 word;
//   * values are packed along tokens: each lane ORs its slot's codes into the
//     words of its 8 channels, the four slots are combined by permlane swaps
//     when a word row is complete, and one slot stores the row (32 bytes per
//     lane); a word row the written range covers only in part is read, merged
//     and written back, so tokens outside the range keep their codes.
// Blocks are 128-token aligned, a multiple of every g and of E = 32/bits, so
// no group and no packed value word is shared by two work-groups.
#include <hip/hip_runtime.h>
#include <math.h>

#include "foscar_internal.h"

namespace foscar {
namespace {

constexpr int kQBlock = 128;  // tokens per work-group

// bf16 -> fp32 as a conversion, not a bit cast: the compiler then knows the values are canonical
// and takes their min / max without canonicalising each one first (same bits, same shift)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return (float)__builtin_bit_cast(__bf16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return (float)__builtin_bit_cast(__bf16, (uint16_t)(w >> 16)); }
__device__ __forceinline__ uint16_t h_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }

// bit offset of element e inside its packed word (even elements in the low
// half-word, odd elements in the high half-word)
template <int BITS>
__device__ __forceinline__ int elem_shift(int e) { return BITS * (e >> 1) + 16 * (e & 1); }

// RN(x / L) for L = 2^BITS - 1 (3 or 15) and x >= 0: q = RN(x * c) with c = RN(1 / L), then one
// correction with the exact remainder, r = fma(-q, L, x), q' = fma(r, c, q) (division by a constant
// with a fused multiply-add, after Markstein).  Checked against the correctly rounded quotient for
// every non-negative finite fp32 x, for both L; x = +inf keeps q (= inf), where r is NaN.
template <int BITS>
__device__ __forceinline__ float div_range(float x) {
  constexpr float L = (float)((1 << BITS) - 1);
  constexpr float c = 1.0f / L;
  const float q = x * c;
  const float q2 = __builtin_fmaf(__builtin_fmaf(-q, L, x), c, q);
  return x == INFINITY ? q : q2;
}

template <int BITS>
struct GroupQ {
  _Float16 s16, z16;
  float s, z;  // fp32 values of s16, z16
  GroupQ() = default;
  __device__ __forceinline__ GroupQ(float mn, float mx) {
    s16 = (_Float16)div_range<BITS>(mx - mn);  // fp32 quotient rounded once, then to fp16 (RNE)
    z16 = (_Float16)mn;
    s = (float)s16;
    z = (float)z16;
  }
  // rint(RN((x - z) / s)), clamped: the correctly rounded division
  __device__ __forceinline__ uint32_t code_exact(float x) const {
    if (s == 0.f) return 0u;
    return (uint32_t)__builtin_amdgcn_fmed3f(rintf(__fdiv_rn(x - z, s)), 0.f, (float)((1 << BITS) - 1));
  }
  __device__ __forceinline__ float rcp() const { return s == 0.f ? 0.f : __builtin_amdgcn_rcpf(s); }
};

// Cross-lane reductions with DPP and permlane swaps (inline asm: a block opens
// with three wait states, which covers a v_dot2 write of its operands as well
// as an ordinary VALU write, and a read inside it follows its write by two).  Every
// step pairs lanes symmetrically (quad xor 1 and 2, half-row and row mirrors,
// row-pair and half-wave swaps), so every lane ends with the result.
#define FOSCAR_DPP_MINMAX(mn, mx, ctrl)                                               \
  asm volatile("s_nop 2\n\t"                                                        \
               "v_min_f32_dpp %0, %0, %0 " ctrl " row_mask:0xf bank_mask:0xf\n\t"   \
               "v_max_f32_dpp %1, %1, %1 " ctrl " row_mask:0xf bank_mask:0xf"         \
               : "+v"(mn), "+v"(mx))
#define FOSCAR_DPP_OR(v, ctrl) \
  asm volatile("s_nop 2\n\tv_or_b32_dpp %0, %0, %0 " ctrl " row_mask:0xf bank_mask:0xf" : "+v"(v))

struct QuantArgs {
  const uint32_t* ksrc;    // bf16 pairs [B][Hkv][N][D/2]
  const uint32_t* vsrc;
  const int32_t* start;    // [B]
  const int32_t* count;    // [B]
  uint32_t* pk;            // [B][Hkv][Tcap][D*bits/32]
  uint32_t* pv;            // [B][Hkv][Tcap*bits/32][D]
  uint16_t* ks;            // fp16 scales / offsets, token-wise [B][Hkv][Tcap][D/g], channel-wise [B][Hkv][Tcap/g][D]
  uint16_t* kz;
  uint16_t* vs;
  uint16_t* vz;
  int32_t hkv, tcap, n_src;
  int32_t rot;             // bit 0: rotate the key rows, bit 1: the value rows (rotate_row8)
};

// Codes of 8 values with scales s[j], offsets z[j] and r[j] = rcp(s[j]) (0
// when s[j] = 0).  rint((x - z) * r) equals rint of the correctly rounded
// quotient RN((x - z) / s) unless the product lies within 2^-16 of a
// half-integer: rcp is within 1 ulp, so the product is within 3 ulp (< 2^-18
// for quotients below 16) of that quotient.  If any lane of the wave has such
// a value, the whole wave recomputes its 8 codes with the correctly rounded
// division (a uniform branch, rarely taken; a per-value select would make the
// compiler run the division every time).
template <int BITS>
__device__ __forceinline__ void code8(const float (&x)[8], const GroupQ<BITS> (&g)[8], const float (&r)[8],
                                      uint32_t (&c)[8]) {
  constexpr float L = (float)((1 << BITS) - 1);
  float dev = 0.f;  // largest distance of a product from its nearest integer (a max, not an OR of
                    // flags: the compiler builds a bit mask out of the flags, ~30 instructions)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float q = (x[j] - g[j].z) * r[j];
    const float k = rintf(q);
    dev = fmaxf(dev, fabsf(q - k));
    c[j] = (uint32_t)__builtin_amdgcn_fmed3f(k, 0.f, L);
  }
  if (__builtin_expect(__any(dev > 0.5f - 0x1p-16f), 0)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = g[j].code_exact(x[j]);
  }
}

// OR / min / max of a value over the four token slots (lanes l, l^16, l^32,
// l^48): v_permlane16_swap pairs rows 0-1 and 2-3, v_permlane32_swap the two
// halves; every lane ends with the result.
__device__ __forceinline__ uint32_t or_slots(uint32_t v) {
  uint32_t a;
  asm volatile(
      "s_nop 2\n\tv_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_or_b32 %0, %0, %1\n\t"
      "v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_or_b32 %0, %0, %1"
      : "+v"(v), "=&v"(a));
  return v;
}
__device__ __forceinline__ void minmax_slots(float& mn, float& mx) {
  float a, b;
  asm volatile(
      "s_nop 2\n\tv_mov_b32 %2, %0\n\tv_mov_b32 %3, %1\n\ts_nop 1\n\t"
      "v_permlane16_swap_b32 %0, %2\n\tv_permlane16_swap_b32 %1, %3\n\t"
      "v_min_f32 %0, %0, %2\n\tv_max_f32 %1, %1, %3\n\t"
      "v_mov_b32 %2, %0\n\tv_mov_b32 %3, %1\n\ts_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %2\n\tv_permlane32_swap_b32 %1, %3\n\t"
      "v_min_f32 %0, %0, %2\n\tv_max_f32 %1, %1, %3"
      : "+v"(mn), "+v"(mx), "=&v"(a), "=&v"(b));
}
// min / max over the aligned groups of LANES (1, 4, 8 or 16) lanes of one token slot
template <int LANES>
__device__ __forceinline__ void octet_group_minmax(float& mn, float& mx) {
  if constexpr (LANES >= 4) {
    FOSCAR_DPP_MINMAX(mn, mx, "quad_perm:[1,0,3,2]");
    FOSCAR_DPP_MINMAX(mn, mx, "quad_perm:[2,3,0,1]");
  }
  if constexpr (LANES >= 8) FOSCAR_DPP_MINMAX(mn, mx, "row_half_mirror");
  if constexpr (LANES >= 16) FOSCAR_DPP_MINMAX(mn, mx, "row_mirror");
}

// Store the value words of channels 8o .. 8o+7 of one word row for the tokens
// of `mask`, keeping the other tokens' codes.
__device__ __forceinline__ void store_value_octet(uint32_t* row, const uint32_t (&acc)[8], uint32_t mask) {
  uint4* p = reinterpret_cast<uint4*>(row);
  uint4 a = make_uint4(acc[0], acc[1], acc[2], acc[3]), b = make_uint4(acc[4], acc[5], acc[6], acc[7]);
  if (mask != 0xFFFFFFFFu) {
    const uint4 oa = p[0], ob = p[1];
    a.x |= oa.x & ~mask; a.y |= oa.y & ~mask; a.z |= oa.z & ~mask; a.w |= oa.w & ~mask;
    b.x |= ob.x & ~mask; b.y |= ob.y & ~mask; b.z |= ob.z & ~mask; b.w |= ob.w & ~mask;
  }
  p[0] = a;
  p[1] = b;
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& w, float (&x)[8]) {
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}

// Rotated cache: the 128 channels of one token row, held 8 per lane (channel
// 8 o + j in x[j], o = lane % 16, the 16 lanes of a token slot), times the
// orthonormal Sylvester-Hadamard matrix H.  Butterflies on the channel index
// bits, 0-2 inside the lane and 3-6 against lanes o ^ 1, 2, 4, 8, in fp64,
// where the sums of bf16 values are exact (rows spanning under 2^38); then
// one scaling by 1/sqrt(128) in fp64 and one rounding to fp32, the precision
// the codes are decided in.
__device__ __forceinline__ void rotate_row8(float (&x)[8], int o) {
  double v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (double)x[j];
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j & h) continue;
      const double a = v[j], b = v[j | h];
      v[j] = a + b;
      v[j | h] = a - b;
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bool upper = (o >> k) & 1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double p = __shfl_xor(v[j], 1 << k);
      v[j] = upper ? p - v[j] : v[j] + p;
    }
  }
  constexpr double kInvSqrt128 = 0x1.6a09e667f3bcdp-4;  // 1/sqrt(128) = sqrt(2)/16, correctly rounded
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)(v[j] * kInvSqrt128);
}

// One side (keys or values) of tokens [t_lo, t_hi) of one (sequence, KV head).
// Lane l works on token slot r = l / 16 of each step of four tokens and on the
// channel octet o = l % 16 (channels 8o .. 8o+7): one 16-byte load per lane
// and row, four consecutive 256-byte rows per wave-instruction.  ROT: the rows
// are rotated (rotate_row8) before they are quantised.
template <int BITS, bool CH, int GRP, bool VALUE, bool ROT>
__device__ __forceinline__ void quant_side(const uint32_t* src, uint32_t* packed, uint16_t* sc, uint16_t* zr,
                                           size_t bh, int tcap, int n_src, int s0, int t_lo, int t_hi) {
  constexpr int D = kHeadDim, E = 32 / BITS, KW = D / E;
  constexpr int L = (1 << BITS) - 1;
  const int lane = threadIdx.x;
  const int r = lane >> 4, o = lane & 15;
  const uint4* src_bh = reinterpret_cast<const uint4*>(src + bh * (size_t)n_src * (D / 2)) + o;  // row t - s0: [(t - s0) * 16]
  uint32_t* vrow = packed + bh * (size_t)(tcap / E) * D + 8 * o;  // value word row w at vrow[w * D]
  const uint32_t cmask = (uint32_t)L;
  // key words: element e of channel 8o + j inside its word
  auto key_word = [&](const uint32_t (&c)[8]) {
    uint32_t part = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = (8 * o + j) % E;
      part |= c[j] << elem_shift<BITS>(e);
    }
    return part;
  };
  auto store_key = [&](int t, bool act, const uint32_t (&c)[8]) {
    uint32_t w = key_word(c);
    if constexpr (BITS == 2) {  // a word is 16 channels: octets 2m and 2m+1
      FOSCAR_DPP_OR(w, "quad_perm:[1,0,3,2]");
      if (act && (o & 1) == 0) packed[(bh * tcap + t) * KW + o / 2] = w;
    } else {  // a word is 8 channels: one octet
      if (act) packed[(bh * tcap + t) * KW + o] = w;
    }
  };
  // value words: token slots of a step share a word row (E is a multiple of 4)
  uint32_t acc[8], msk = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0;
  auto add_value = [&](int t, bool act, const uint32_t (&c)[8]) {
    const int sh = elem_shift<BITS>(t % E);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] |= c[j] << sh;
    msk |= act ? (cmask << sh) : 0u;
  };
  auto flush_value = [&](int tb) {  // word row of the step starting at tb
    // slots past the range were coded from zero rows: keep the written tokens' bits only
    msk = or_slots(msk);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = or_slots(acc[j]) & msk;
    if (r == 0 && msk != 0) store_value_octet(vrow + (size_t)(tb / E) * D, acc, msk);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0;
    msk = 0;
  };
  // Steps of four tokens from t_lo rounded down to 4; rows are loaded U steps
  // ahead (the cross-lane asm keeps the compiler from hoisting later loads).
  constexpr int U = 4;
  auto load_steps = [&](uint4 (&w)[U], int tb, int t_a, int t_b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tb + 4 * u + r;
      w[u] = (t >= t_a && t < t_b) ? src_bh[(size_t)(t - s0) * 16] : make_uint4(0, 0, 0, 0);
    }
  };

  if constexpr (!CH) {
    const int t_first = t_lo & ~3;
    for (int tb0 = t_first; tb0 < t_hi; tb0 += 4 * U) {
      uint4 wb[U];
      load_steps(wb, tb0, t_lo, t_hi);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int tb = tb0 + 4 * u;
        if (tb >= t_hi) break;
        const int t = tb + r;
        const bool act = t >= t_lo && t < t_hi;
        float x[8];
        unpack_bf16x8(wb[u], x);
        if constexpr (ROT) rotate_row8(x, o);
        float mn = fminf(fminf(fminf(x[0], x[1]), fminf(x[2], x[3])), fminf(fminf(x[4], x[5]), fminf(x[6], x[7])));
        float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        octet_group_minmax<GRP / 8>(mn, mx);  // the g/8 lanes of this lane's group
        const GroupQ<BITS> gq(mn, mx);
        const float rq = gq.rcp();
        if (act && (8 * o) % GRP == 0) {
          const size_t si = (bh * tcap + t) * (D / GRP) + (8 * o) / GRP;
          sc[si] = h_bits(gq.s16);
          zr[si] = h_bits(gq.z16);
        }
        const GroupQ<BITS> gs[8] = {gq, gq, gq, gq, gq, gq, gq, gq};
        const float rs[8] = {rq, rq, rq, rq, rq, rq, rq, rq};
        uint32_t c[8];
        code8<BITS>(x, gs, rs, c);
        if constexpr (!VALUE) {
          store_key(t, act, c);
        } else {
          add_value(t, act, c);
          if ((tb + 4) % E == 0 || tb + 4 >= t_hi) flush_value(tb);
        }
      }
    }
  } else {
    // channel-wise groups: [g0, g0 + GRP) from token 0; t_lo is a group start (a multiple of 4)
    for (int g0 = t_lo; g0 < t_hi; g0 += GRP) {
      const int g1 = min(g0 + GRP, t_hi);
      float mn[8], mx[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        mn[j] = INFINITY;
        mx[j] = -INFINITY;
      }
      for (int tb0 = g0; tb0 < g1; tb0 += 4 * U) {
        uint4 wb[U];
        load_steps(wb, tb0, g0, g1);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (tb0 + 4 * u + r >= g1) continue;  // this slot's token is past the group (lane-local)
          float x[8];
          unpack_bf16x8(wb[u], x);
          if constexpr (ROT) rotate_row8(x, o);  // (the 16 lanes of a slot skip or run together)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            mn[j] = fminf(mn[j], x[j]);
            mx[j] = fmaxf(mx[j], x[j]);
          }
        }
      }
      GroupQ<BITS> gq[8];
      float rc[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        minmax_slots(mn[j], mx[j]);
        gq[j] = GroupQ<BITS>(mn[j], mx[j]);
        rc[j] = gq[j].rcp();
      }
      if (r == 0) {
        const size_t si = (bh * (size_t)(tcap / GRP) + g0 / GRP) * D + 8 * o;
        uint4 sv, zv;
        auto pair = [&](const _Float16& a, const _Float16& b) { return (uint32_t)h_bits(a) | ((uint32_t)h_bits(b) << 16); };
        sv = make_uint4(pair(gq[0].s16, gq[1].s16), pair(gq[2].s16, gq[3].s16), pair(gq[4].s16, gq[5].s16),
                        pair(gq[6].s16, gq[7].s16));
        zv = make_uint4(pair(gq[0].z16, gq[1].z16), pair(gq[2].z16, gq[3].z16), pair(gq[4].z16, gq[5].z16),
                        pair(gq[6].z16, gq[7].z16));
        *reinterpret_cast<uint4*>(sc + si) = sv;
        *reinterpret_cast<uint4*>(zr + si) = zv;
      }
      for (int tb0 = g0; tb0 < g1; tb0 += 4 * U) {
        uint4 wb[U];
        load_steps(wb, tb0, g0, g1);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int tb = tb0 + 4 * u;
          if (tb >= g1) break;
          const int t = tb + r;
          const bool act = t < g1;
          float x[8];
          unpack_bf16x8(wb[u], x);
          if constexpr (ROT) rotate_row8(x, o);
          uint32_t c[8];
          code8<BITS>(x, gq, rc, c);
          if constexpr (!VALUE) {
            store_key(t, act, c);
          } else {
            add_value(t, act, c);
            if ((tb + 4) % E == 0 || tb + 4 >= g1) flush_value(tb);
          }
        }
      }
    }
  }
}

template <int BITS, bool KCH, bool VCH, int GRP>
__global__ __launch_bounds__(64) void quant_append(const QuantArgs a) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int s0 = a.start[b];
  if (s0 < 0 || s0 > a.tcap) return;               // out of range: the sequence is left as it is
  if ((KCH || VCH) && s0 % GRP != 0) return;       // a channel-wise side starts at a group boundary
  const int n = min(max(a.count[b], 0), min(a.n_src, a.tcap - s0));
  const int blk = (s0 / kQBlock + (int)blockIdx.x) * kQBlock;
  const int t_lo = max(blk, s0), t_hi = min(blk + kQBlock, s0 + n);
  if (t_lo >= t_hi) return;
  const size_t bh = (size_t)b * a.hkv + h;
  if (a.rot & 1)
    quant_side<BITS, KCH, GRP, false, true>(a.ksrc, a.pk, a.ks, a.kz, bh, a.tcap, a.n_src, s0, t_lo, t_hi);
  else
    quant_side<BITS, KCH, GRP, false, false>(a.ksrc, a.pk, a.ks, a.kz, bh, a.tcap, a.n_src, s0, t_lo, t_hi);
  if (a.rot & 2)
    quant_side<BITS, VCH, GRP, true, true>(a.vsrc, a.pv, a.vs, a.vz, bh, a.tcap, a.n_src, s0, t_lo, t_hi);
  else
    quant_side<BITS, VCH, GRP, true, false>(a.vsrc, a.pv, a.vs, a.vz, bh, a.tcap, a.n_src, s0, t_lo, t_hi);
}

template <int BITS, bool KCH, bool VCH>
hipError_t launch_g(int group, dim3 grid, const QuantArgs& a, hipStream_t st) {
  switch (group) {
    case 32: hipLaunchKernelGGL((quant_append<BITS, KCH, VCH, 32>), grid, dim3(64), 0, st, a); break;
    case 64: hipLaunchKernelGGL((quant_append<BITS, KCH, VCH, 64>), grid, dim3(64), 0, st, a); break;
    case 128: hipLaunchKernelGGL((quant_append<BITS, KCH, VCH, 128>), grid, dim3(64), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(bool kch, bool vch, int group, dim3 grid, const QuantArgs& a, hipStream_t st) {
  if (kch) return vch ? launch_g<BITS, true, true>(group, grid, a, st) : launch_g<BITS, true, false>(group, grid, a, st);
  return vch ? launch_g<BITS, false, true>(group, grid, a, st) : launch_g<BITS, false, false>(group, grid, a, st);
}

}  // namespace

hipError_t launch_quantize(int bits, bool k_channel, bool v_channel, int group, int rot, int batch, int hkv, int tcap,
                           int n_src, const void* k_src, const void* v_src, const int32_t* start, const int32_t* count,
                           void* pk, void* pv, void* ks, void* kz, void* vs, void* vz, hipStream_t stream) {
  QuantArgs a;
  a.rot = rot;
  a.ksrc = (const uint32_t*)k_src;
  a.vsrc = (const uint32_t*)v_src;
  a.start = start;
  a.count = count;
  a.pk = (uint32_t*)pk;
  a.pv = (uint32_t*)pv;
  a.ks = (uint16_t*)ks;
  a.kz = (uint16_t*)kz;
  a.vs = (uint16_t*)vs;
  a.vz = (uint16_t*)vz;
  a.hkv = hkv;
  a.tcap = tcap;
  a.n_src = n_src;
  // a range of n_src tokens that starts inside a block touches one block more
  const dim3 grid((unsigned)((n_src + kQBlock - 1) / kQBlock + 1), (unsigned)hkv, (unsigned)batch);
  if (bits == 2) return launch_bits<2>(k_channel, v_channel, group, grid, a, stream);
  return launch_bits<4>(k_channel, v_channel, group, grid, a, stream);
}

}  // namespace foscar
