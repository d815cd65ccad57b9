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
// Work decomposition: one wave per (128-token block, KV head, sequence).
// Lane l owns channels 2l and 2l+1 of each token row (one 4-byte bf16 pair
// per row, so a row is one 256-byte coalesced load).
//   * token-wise group (g channels of a token = g/2 lanes): min / max by
//     xor-shuffles inside the g/2 lanes;
//   * channel-wise group (g tokens of a channel): each lane folds the group's
//     tokens into its two channels' min / max, then codes them on a second
//     pass (the group's rows are re-read, from L2);
//   * keys are packed along channels: the E/2 lanes of a word OR their codes
//     together by xor-shuffles and one lane stores the word;
//   * values are packed along tokens: each lane gathers the E tokens of its
//     two channels' words in registers and stores them as one 8-byte write;
//     a word that the written range covers only in part is read, merged and
//     written back, so tokens outside the range keep their codes.
// Blocks are 128-token aligned, a multiple of every g and of E = 32/bits, so
// no group and no packed value word is shared by two work-groups.
#include <hip/hip_runtime.h>
#include <math.h>

#include "foscar_internal.h"

namespace foscar {
namespace {

constexpr int kQBlock = 128;  // tokens per work-group

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint16_t h_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }

// bit offset of element e inside its packed word (even elements in the low
// half-word, odd elements in the high half-word)
template <int BITS>
__device__ __forceinline__ int elem_shift(int e) { return BITS * (e >> 1) + 16 * (e & 1); }

template <int BITS>
struct GroupQ {
  _Float16 s16, z16;
  float s, z;  // fp32 values of s16, z16
  __device__ __forceinline__ GroupQ(float mn, float mx) {
    constexpr float L = (float)((1 << BITS) - 1);
    s16 = (_Float16)__fdiv_rn(mx - mn, L);  // fp32 quotient rounded once, then to fp16 (RNE)
    z16 = (_Float16)mn;
    s = (float)s16;
    z = (float)z16;
  }
  // rint(RN(d / s)) for d = x - z: with r = rcp(s) (1 ulp), d * r lies within
  // 3 ulp of the correctly rounded quotient, so its nearest integer is the same
  // unless it sits within that distance of a half-integer; |quotient| < 16
  // there, where 2^-16 is many ulps.  Only those rare lanes take the exact
  // division.
  __device__ __forceinline__ uint32_t code(float x, float r) const {
    if (s == 0.f) return 0u;
    const float d = x - z;
    float q = d * r;
    const float f = q - floorf(q);
    if (fabsf(f - 0.5f) < 0x1p-16f) q = __fdiv_rn(d, s);
    q = rintf(q);  // round half to even
    return (uint32_t)fminf(fmaxf(q, 0.f), (float)((1 << BITS) - 1));
  }
  __device__ __forceinline__ float rcp() const { return s == 0.f ? 0.f : __builtin_amdgcn_rcpf(s); }
};

// Cross-lane reductions with DPP and permlane swaps (inline asm: each
// cross-lane read of a VGPR follows its VALU write by two wait states).  Every
// step pairs lanes symmetrically (quad xor 1 and 2, half-row and row mirrors,
// row-pair and half-wave swaps), so every lane ends with the result.
#define FOSCAR_DPP_MINMAX(mn, mx, ctrl)                                               \
  asm volatile("s_nop 1\n\t"                                                        \
               "v_min_f32_dpp %0, %0, %0 " ctrl " row_mask:0xf bank_mask:0xf\n\t"   \
               "v_max_f32_dpp %1, %1, %1 " ctrl " row_mask:0xf bank_mask:0xf"         \
               : "+v"(mn), "+v"(mx))
#define FOSCAR_DPP_OR(v, ctrl) \
  asm volatile("s_nop 1\n\tv_or_b32_dpp %0, %0, %0 " ctrl " row_mask:0xf bank_mask:0xf" : "+v"(v))

// min and max over each aligned group of LANES lanes (16, 32 or 64)
template <int LANES>
__device__ __forceinline__ void group_minmax(float& mn, float& mx) {
  FOSCAR_DPP_MINMAX(mn, mx, "quad_perm:[1,0,3,2]");
  FOSCAR_DPP_MINMAX(mn, mx, "quad_perm:[2,3,0,1]");
  FOSCAR_DPP_MINMAX(mn, mx, "row_half_mirror");
  FOSCAR_DPP_MINMAX(mn, mx, "row_mirror");
  if constexpr (LANES >= 32) {
    float a, b;
    asm volatile(
        "v_mov_b32 %2, %0\n\tv_mov_b32 %3, %1\n\ts_nop 1\n\t"
        "v_permlane16_swap_b32 %0, %2\n\tv_permlane16_swap_b32 %1, %3\n\t"
        "v_min_f32 %0, %0, %2\n\tv_max_f32 %1, %1, %3"
        : "+v"(mn), "+v"(mx), "=&v"(a), "=&v"(b));
  }
  if constexpr (LANES == 64) {
    float a, b;
    asm volatile(
        "v_mov_b32 %2, %0\n\tv_mov_b32 %3, %1\n\ts_nop 1\n\t"
        "v_permlane32_swap_b32 %0, %2\n\tv_permlane32_swap_b32 %1, %3\n\t"
        "v_min_f32 %0, %0, %2\n\tv_max_f32 %1, %1, %3"
        : "+v"(mn), "+v"(mx), "=&v"(a), "=&v"(b));
  }
}

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
};

// OR of `v` over the E/2 lanes (4 or 8, aligned) that share one key word
template <int BITS>
__device__ __forceinline__ uint32_t or_word_lanes(uint32_t v) {
  FOSCAR_DPP_OR(v, "quad_perm:[1,0,3,2]");
  FOSCAR_DPP_OR(v, "quad_perm:[2,3,0,1]");
  if constexpr (BITS == 2) FOSCAR_DPP_OR(v, "row_half_mirror");
  return v;
}

// Store the value words of channels 2*lane, 2*lane+1 for the tokens of `mask`
// (word row `row`), keeping the other tokens' codes.
__device__ __forceinline__ void store_value_words(uint32_t* pv_row, uint32_t acc0, uint32_t acc1, uint32_t mask) {
  uint2* p = reinterpret_cast<uint2*>(pv_row);
  if (mask != 0xFFFFFFFFu) {
    const uint2 old = *p;
    acc0 |= old.x & ~mask;
    acc1 |= old.y & ~mask;
  }
  *p = make_uint2(acc0, acc1);
}

// One side (keys or values) of tokens [t_lo, t_hi) of one (sequence, KV head).
template <int BITS, bool CH, int GRP, bool VALUE>
__device__ __forceinline__ void quant_side(const uint32_t* src, uint32_t* packed, uint16_t* sc, uint16_t* zr,
                                           size_t bh, int tcap, int n_src, int s0, int t_lo, int t_hi) {
  constexpr int D = kHeadDim, E = 32 / BITS, KW = D / E;
  const int lane = threadIdx.x;
  const uint32_t* src_bh = src + bh * (size_t)n_src * (D / 2) + lane;  // token t is source row t - s0
  auto load_row = [&](int t) { return src_bh[(size_t)(t - s0) * (D / 2)]; };
  const uint32_t cmask = (1u << BITS) - 1u;
  const int e0 = (2 * lane) % E;  // element of channel 2*lane inside its key word (even)
  auto store_key = [&](int t, uint32_t c0, uint32_t c1) {
    const uint32_t w = or_word_lanes<BITS>((c0 << elem_shift<BITS>(e0)) | (c1 << elem_shift<BITS>(e0 + 1)));
    if (lane % (E / 2) == 0) packed[(bh * tcap + t) * KW + (2 * lane) / E] = w;
  };
  uint32_t* vrow = packed + bh * (size_t)(tcap / E) * D + 2 * lane;  // value word row r at vrow[r * D]
  // Rows are loaded U at a time ahead of their processing: the cross-lane asm
  // of the processing keeps the compiler from moving later loads above it,
  // which would leave one row load in flight per wave.
  constexpr int U = 16;
  auto load_batch = [&](uint32_t(&w)[U], int t, int t_end) {
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = (t + u < t_end) ? load_row(t + u) : 0u;
  };

  if constexpr (!CH) {
    uint32_t acc0 = 0, acc1 = 0, msk = 0;
    for (int tb = t_lo; tb < t_hi; tb += U) {
     uint32_t wb[U];
     load_batch(wb, tb, t_hi);
#pragma unroll
     for (int u = 0; u < U; ++u) {
      const int t = tb + u;
      if (t >= t_hi) break;
      const uint32_t w = wb[u];
      const float x0 = bf16_lo(w), x1 = bf16_hi(w);
      float mn = fminf(x0, x1), mx = fmaxf(x0, x1);
      group_minmax<GRP / 2>(mn, mx);  // the g/2 lanes of this lane's group
      const GroupQ<BITS> gq(mn, mx);
      const float rq = gq.rcp();
      if ((2 * lane) % GRP == 0) {
        const size_t si = (bh * tcap + t) * (D / GRP) + (2 * lane) / GRP;
        sc[si] = h_bits(gq.s16);
        zr[si] = h_bits(gq.z16);
      }
      const uint32_t c0 = gq.code(x0, rq), c1 = gq.code(x1, rq);
      if constexpr (!VALUE) {
        store_key(t, c0, c1);
      } else {
        const int sh = elem_shift<BITS>(t % E);
        acc0 |= c0 << sh;
        acc1 |= c1 << sh;
        msk |= cmask << sh;
        if (t % E == E - 1 || t == t_hi - 1) {
          store_value_words(vrow + (size_t)(t / E) * D, acc0, acc1, msk);
          acc0 = acc1 = msk = 0;
        }
      }
     }
    }
  } else {
    // channel-wise groups: [g0, g0 + GRP) from token 0; t_lo is a group start
    for (int g0 = t_lo; g0 < t_hi; g0 += GRP) {
      const int g1 = min(g0 + GRP, t_hi);
      float mn0 = INFINITY, mx0 = -INFINITY, mn1 = INFINITY, mx1 = -INFINITY;
#pragma unroll 8
      for (int t = g0; t < g1; ++t) {
        const uint32_t w = load_row(t);
        const float x0 = bf16_lo(w), x1 = bf16_hi(w);
        mn0 = fminf(mn0, x0);
        mx0 = fmaxf(mx0, x0);
        mn1 = fminf(mn1, x1);
        mx1 = fmaxf(mx1, x1);
      }
      const GroupQ<BITS> q0(mn0, mx0), q1(mn1, mx1);
      const float r0 = q0.rcp(), r1 = q1.rcp();
      const size_t si = (bh * (size_t)(tcap / GRP) + g0 / GRP) * D + 2 * lane;
      *reinterpret_cast<uint32_t*>(sc + si) = (uint32_t)h_bits(q0.s16) | ((uint32_t)h_bits(q1.s16) << 16);
      *reinterpret_cast<uint32_t*>(zr + si) = (uint32_t)h_bits(q0.z16) | ((uint32_t)h_bits(q1.z16) << 16);
      uint32_t acc0 = 0, acc1 = 0, msk = 0;
      for (int tb = g0; tb < g1; tb += U) {
       uint32_t wb[U];
       load_batch(wb, tb, g1);
#pragma unroll
       for (int u = 0; u < U; ++u) {
        const int t = tb + u;
        if (t >= g1) break;
        const uint32_t w = wb[u];
        const uint32_t c0 = q0.code(bf16_lo(w), r0), c1 = q1.code(bf16_hi(w), r1);
        if constexpr (!VALUE) {
          store_key(t, c0, c1);
        } else {
          const int sh = elem_shift<BITS>(t % E);
          acc0 |= c0 << sh;
          acc1 |= c1 << sh;
          msk |= cmask << sh;
          if (t % E == E - 1 || t == g1 - 1) {
            store_value_words(vrow + (size_t)(t / E) * D, acc0, acc1, msk);
            acc0 = acc1 = msk = 0;
          }
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
  quant_side<BITS, KCH, GRP, false>(a.ksrc, a.pk, a.ks, a.kz, bh, a.tcap, a.n_src, s0, t_lo, t_hi);
  quant_side<BITS, VCH, GRP, true>(a.vsrc, a.pv, a.vs, a.vz, bh, a.tcap, a.n_src, s0, t_lo, t_hi);
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

hipError_t launch_quantize(int bits, bool k_channel, bool v_channel, int group, int batch, int hkv, int tcap,
                           int n_src, const void* k_src, const void* v_src, const int32_t* start, const int32_t* count,
                           void* pk, void* pv, void* ks, void* kz, void* vs, void* vz, hipStream_t stream) {
  QuantArgs a;
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
