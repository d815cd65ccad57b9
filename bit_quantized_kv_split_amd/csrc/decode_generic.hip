// Decode attention for head dimensions other than 128 (a multiple of 32 up to
// 256), over the same packed caches and with the same folds as the D = 128
// kernels: keys packed along channels, values along tokens, one fp16 (scale,
// offset) pair per group, token-wise or channel-wise on either side.
//
// FOSCAR explainer ("FOSCAR speeds up 2-bit KV decode"), fold-placement table
// and fold-rule paragraph:
//   token-wise K   (acc-fold):     score += s_tj * sum_{c in j} q_c code_c + z_tj * sum_{c in j} q_c
//   channel-wise K (operand-fold): q~_c = q_c s_tau,c once per token group tau; score = q~ . code + sum_c q_c z_tau,c
//   token-wise V   (operand-fold): p~_tj = p_t s_tj; out_c += p~_t,j(c) code_t,c, plus sum_t p_t z_t,j(c)
//   channel-wise V (acc-fold):     out_c += s_tau,c * sum_{t in tau} p_t code_t,c + z_tau,c * sum_{t in tau} p_t
// Key-side terms enter the score before the softmax; value-side terms enter
// the weighted sum before the division by the softmax denominator.
//
// Two launches: gd_split gives each (work pair, token range) a work-group that
// writes the range's normalised output and natural-log lse (one work pair is
// a KV head's group of at most four query heads); gd_merge combines the
// ranges of each query row by log-sum-exp into bf16 out and fp32 lse.
//
// Layout of the work: the 4 waves of a work-group take the range's 64-token
// blocks in turn.  Scores have lane = token (the lane walks its token's key
// words a channel group at a time, the next group's words in flight; the
// query operand is an LDS broadcast), the online softmax reduces over the
// wave, and the weighted values have lane = channel (64 consecutive channels
// per pass, so each value-word load is one coalesced row segment; a block's
// word rows one at a time, every pass's word of a row loaded together, the
// next row in flight).  Every step runs on the vector ALUs (fp16 dot products
// of code pairs where the operand allows, fp32 FMAs for q * s of channel-wise
// keys).  Tokens at or past the sequence length are never loaded.
#include "foscar_internal.h"

namespace foscar {

namespace {

constexpr int kGdThreads = 256;
constexpr int kGdWaves = kGdThreads / 64;
constexpr int kGdPass = kGdMaxD / 64;  // channels per lane in the value pass

__device__ __forceinline__ float half_to_float(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ float bf16_to_float(uint16_t h) { return __builtin_bit_cast(float, (uint32_t)h << 16); }

__device__ __forceinline__ uint16_t float_to_bf16(float f) {  // round to nearest even
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ int elem_shift(int bits, int e) { return bits * (e >> 1) + 16 * (e & 1); }

// Wave reductions: DPP within each row of 16 lanes (quad_perm [1,0,3,2] and
// [2,3,0,1], then row rotations by 4 and 8 leave every lane of a row with the
// row's result), then the four rows' results read as scalars; the result is
// wave-uniform.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x124>(v);
  v += dpp<0x128>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x124>(v));
  v = fmaxf(v, dpp<0x128>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// LDS written by some lanes of a wave and read by others of the same wave
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct alignas(16) F4 {
  float v[kMaxG];
};

// Code pairs as fp16 operands: the two codes of elements 2k and 2k+1 of a word
// sit at bits bits*k and 16 + bits*k, so one shift and one AND give them as the
// bit patterns of two fp16 subnormals, exactly code * 2^-24 each (no bias to
// take back).  v_dot2_f32_f16 multiplies them with a pair of fp16 operands
// (query channels, or softmax weights) and accumulates in fp32; the sum is
// scaled by 2^24 once per group.
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
constexpr float kCodeScale = 16777216.0f;  // 2^24
__device__ __forceinline__ float dot2(uint32_t a, uint32_t codes, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, codes), c, false);
}
__device__ __forceinline__ uint16_t f16_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

extern __shared__ F4 s_dyn[];  // launch-sized LDS: kGdWaves * 2 * D entries for channel-wise keys, else none

template <int BITS, bool KCH, bool VCH, int GRP>
__global__ __launch_bounds__(kGdThreads) void gd_split(const GenericArgs a) {
  constexpr int E = 32 / BITS;
  constexpr int g = GRP;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  constexpr uint32_t PMASK = MASK | (MASK << 16);  // a code pair
  const int D = a.d, G = a.g_heads, S = a.splits;
  const int pair = blockIdx.x, s = blockIdx.y;
  const int b = pair / a.pairs, pp = pair - b * a.pairs;
  const int kvh = pp / a.kv_group;  // KV head; query heads h0 .. h0 + G - 1
  const int h0 = pp * G;
  const int T = min(max(a.seq_lens[b], 0), a.tcap);
  const int r0 = s * a.chunk, r1 = min(r0 + a.chunk, T);
  const size_t bh = (size_t)b * a.hkv + kvh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int W = D / E;   // key words per token
  const int NJ = D / g;  // channel groups of a token (token-wise sides)

  __shared__ F4 s_q[kGdMaxD];                                   // q[h][c] as [c][h]
  __shared__ uint4 s_q2[kGdMaxD / 2];                           // fp16 pairs (q[h][2i], q[h][2i+1]), h = x, y, z, w
  __shared__ float s_qsum[kGdMaxD / 32][kMaxG];                 // token-wise K: sum of q over channel group j
  F4* const s_qt = s_dyn;  // channel-wise K: q~ of a block's (<= 2) token groups, [wave][2][D] (dynamic LDS)
  __shared__ float s_bias[kGdWaves][2][kMaxG];                  // channel-wise K: sum_c q z of those groups
  // fp16 weight pairs of a block (per token pair: 4 heads x (even token, odd token)), per channel
  // group for a token-wise value side; after the loop, the combine o[w][c] (heads in F4)
  constexpr int kWSize = VCH ? kGdWaves * 32 : kGdWaves * (kGdMaxD / 32) * 32;
  constexpr int kOSize = kGdWaves * kGdMaxD;
  __shared__ uint4 s_buf[kWSize > kOSize ? kWSize : kOSize];
  __shared__ float s_zs[kGdWaves][kGdMaxD / 32][kMaxG];         // token-wise V: sum_t p z per channel group
  __shared__ float s_m[kGdWaves][kMaxG], s_l[kGdWaves][kMaxG];

  for (int i = tid; i < D; i += kGdThreads) {
    F4 f;
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) f.v[h] = h < G ? bf16_to_float(a.q[((size_t)b * a.hq + h0 + h) * D + i]) : 0.f;
    s_q[i] = f;
  }
  for (int i = tid; i < D / 2; i += kGdThreads) {
    uint32_t v[kMaxG];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      const size_t r = ((size_t)b * a.hq + h0 + h) * D + 2 * i;
      v[h] = h < G ? (uint32_t)f16_bits(bf16_to_float(a.q[r])) | (uint32_t)f16_bits(bf16_to_float(a.q[r + 1])) << 16
                   : 0u;
    }
    s_q2[i] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  __syncthreads();
  if (!KCH && tid < NJ * kMaxG) {
    const int j = tid / kMaxG, h = tid - j * kMaxG;
    float acc = 0.f;
    for (int c = j * g; c < j * g + g; ++c) acc += s_q[c].v[h];
    s_qsum[j][h] = acc;
  }
  __syncthreads();

  float m[kMaxG], l[kMaxG], o[kGdPass][kMaxG];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < kGdPass; ++i) o[i][h] = 0.f;
  }

  for (int blk = r0 + wave * 64; blk < r1; blk += kGdThreads) {
    const int t = blk + lane;
    const bool valid = t < r1;
    const int tau0 = blk / g;
    constexpr int ntau = (KCH || VCH) && GRP < 64 ? 2 : 1;  // token groups a 64-token block meets (blocks start at
                                                          // multiples of 64)
    constexpr int VW = 64 / E;  // value word rows of a block
    const int tw0 = blk / E, tw1 = min(blk + 64, r1);  // rows tw0 + k hold tokens below tw1 while (tw0 + k) * E < tw1

    // ---- channel-wise K: q~ and the bias of the block's token groups
    if (KCH) {
      for (int u = 0; u < ntau; ++u) {
        const int tau = tau0 + u;
        F4 bias;
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) bias.v[h] = 0.f;
        if (tau * g < r1) {
          for (int c = lane; c < D; c += 64) {
            const size_t si = (bh * (size_t)(a.tcap / g) + tau) * D + c;
            const float sk = half_to_float(a.ks[si]), zk = half_to_float(a.kz[si]);
            const F4 qc = s_q[c];
            F4 qt;
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) {
              qt.v[h] = qc.v[h] * sk;
              bias.v[h] += qc.v[h] * zk;
            }
            s_qt[(wave * 2 + u) * D + c] = qt;
          }
        }
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
          const float bs = wave_sum(bias.v[h]);
          if (lane == 0) s_bias[wave][u][h] = bs;
        }
      }
      wave_lds_sync();
    }

    // ---- scores, lane = token
    float sc[kMaxG];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) sc[h] = 0.f;
    if (valid) {
      const uint32_t* krow = a.pk + (bh * a.tcap + t) * (size_t)W;
      if (KCH) {
        const int u = t / g - tau0;
        const F4* qt = s_qt + (wave * 2 + u) * D;
        uint2 nxt = *reinterpret_cast<const uint2*>(krow);  // W is even: word pairs, the next one in flight
        for (int w = 0; w < W; w += 2) {
          const uint2 cur = nxt;
          if (w + 2 < W) nxt = *reinterpret_cast<const uint2*>(krow + w + 2);
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const uint32_t word = half ? cur.y : cur.x;
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const float cf = (float)((word >> elem_shift(BITS, e)) & MASK);
              const F4 qv = qt[(w + half) * E + e];
#pragma unroll
              for (int h = 0; h < kMaxG; ++h) sc[h] = __builtin_fmaf(qv.v[h], cf, sc[h]);
            }
          }
        }
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) sc[h] += s_bias[wave][u][h];
      } else {
        constexpr int WPG = GRP / E;  // words of a channel group (even)
        uint32_t nxt[WPG];            // the next group's words, in flight while this group is summed
#pragma unroll
        for (int w = 0; w < WPG; w += 2) {
          const uint2 v = *reinterpret_cast<const uint2*>(krow + w);
          nxt[w] = v.x;
          nxt[w + 1] = v.y;
        }
        for (int j = 0; j < NJ; ++j) {
          uint32_t cur[WPG];
#pragma unroll
          for (int w = 0; w < WPG; ++w) cur[w] = nxt[w];
          if (j + 1 < NJ) {
#pragma unroll
            for (int w = 0; w < WPG; w += 2) {
              const uint2 v = *reinterpret_cast<const uint2*>(krow + (j + 1) * WPG + w);
              nxt[w] = v.x;
              nxt[w + 1] = v.y;
            }
          }
          const size_t si = (bh * a.tcap + t) * (size_t)NJ + j;
          const float sk = half_to_float(a.ks[si]), zk = half_to_float(a.kz[si]);
          float acc[kMaxG];
#pragma unroll
          for (int h = 0; h < kMaxG; ++h) acc[h] = 0.f;
#pragma unroll
          for (int w = 0; w < WPG; ++w) {
#pragma unroll
            for (int k = 0; k < E / 2; ++k) {
              const uint32_t cp = (cur[w] >> (BITS * k)) & PMASK;
              const uint4 q4 = s_q2[(j * WPG + w) * (E / 2) + k];
              acc[0] = dot2(q4.x, cp, acc[0]);
              acc[1] = dot2(q4.y, cp, acc[1]);
              acc[2] = dot2(q4.z, cp, acc[2]);
              acc[3] = dot2(q4.w, cp, acc[3]);
            }
          }
#pragma unroll
          for (int h = 0; h < kMaxG; ++h) sc[h] += sk * (acc[h] * kCodeScale) + zk * s_qsum[j][h];
        }
      }
    }

    // ---- online softmax over the block (scores in log2 units)
    float p[kMaxG], alpha[kMaxG];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      const float x = valid ? sc[h] * a.sm_log2 : -INFINITY;
      const float m_new = fmaxf(m[h], wave_max(x));
      if (m_new == -INFINITY) {
        alpha[h] = 1.f;
        p[h] = 0.f;
      } else {
        alpha[h] = exp2f(m[h] - m_new);
        p[h] = valid ? exp2f(x - m_new) : 0.f;
      }
      l[h] = l[h] * alpha[h] + wave_sum(p[h]);
      m[h] = m_new;
    }

    // ---- weights of the block into LDS, lane = token
    float psum[2][kMaxG];
    if (VCH) {
      uint16_t* w16 = reinterpret_cast<uint16_t*>(s_buf + wave * 32) + (lane >> 1) * 8 + (lane & 1);
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) w16[2 * h] = f16_bits(p[h]);
      const int u = ntau == 2 ? (lane >> 5) : 0;
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) {
        psum[0][h] = wave_sum(u == 0 ? p[h] : 0.f);
        psum[1][h] = ntau == 2 ? wave_sum(u == 1 ? p[h] : 0.f) : 0.f;
      }
    } else {
      for (int j = 0; j < NJ; ++j) {
        float sv = 0.f, zv = 0.f;
        if (valid) {
          const size_t si = (bh * a.tcap + t) * (size_t)NJ + j;
          sv = half_to_float(a.vs[si]);
          zv = half_to_float(a.vz[si]);
        }
        uint16_t* w16 =
            reinterpret_cast<uint16_t*>(s_buf + (wave * (kGdMaxD / 32) + j) * 32) + (lane >> 1) * 8 + (lane & 1);
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
          w16[2 * h] = f16_bits(p[h] * sv);
          const float zs = wave_sum(p[h] * zv);
          if (lane == 0) s_zs[wave][j][h] = zs;
        }
      }
    }
    wave_lds_sync();

    // ---- weighted values, lane = channel (channels lane + 64 i): one word row of the block at a
    // time, the row's words of every pass loaded together and the next row in flight
    float accv[kGdPass][kMaxG], part1[kGdPass][kMaxG];  // (channel-wise V, g = 32: tokens 0-31, 32-63)
#pragma unroll
    for (int i = 0; i < kGdPass; ++i)
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) {
        o[i][h] *= alpha[h];
        accv[i][h] = part1[i][h] = 0.f;
      }
    const uint32_t* vbase = a.pv + (bh * (size_t)(a.tcap / E) + tw0) * D + lane;
    uint32_t nv[kGdPass];
#pragma unroll
    for (int i = 0; i < kGdPass; ++i) nv[i] = lane + 64 * i < D ? vbase[64 * i] : 0u;  // row tw0 holds token blk < tw1
    for (int k = 0; k < VW; ++k) {
      if ((tw0 + k) * E >= tw1) break;  // rows past the length
      uint32_t cv[kGdPass];
#pragma unroll
      for (int i = 0; i < kGdPass; ++i) cv[i] = nv[i];
      if ((tw0 + k + 1) * E < tw1 && k + 1 < VW) {
#pragma unroll
        for (int i = 0; i < kGdPass; ++i) nv[i] = lane + 64 * i < D ? vbase[(size_t)(k + 1) * D + 64 * i] : 0u;
      }
      const int lp = k * (E / 2);  // token pair of the row's first two tokens (0 .. 31)
#pragma unroll
      for (int i = 0; i < kGdPass; ++i) {
        const int c = lane + 64 * i;
        if (c < D) {
          const uint4* wp = VCH ? s_buf + wave * 32 + lp : s_buf + (wave * (kGdMaxD / 32) + c / g) * 32 + lp;
          float a4[kMaxG];
#pragma unroll
          for (int h = 0; h < kMaxG; ++h) a4[h] = 0.f;
#pragma unroll
          for (int kk = 0; kk < E / 2; ++kk) {
            const uint32_t cp = (cv[i] >> (BITS * kk)) & PMASK;
            const uint4 w4 = wp[kk];  // weights past the length are zero
            a4[0] = dot2(w4.x, cp, a4[0]);
            a4[1] = dot2(w4.y, cp, a4[1]);
            a4[2] = dot2(w4.z, cp, a4[2]);
            a4[3] = dot2(w4.w, cp, a4[3]);
          }
          if (VCH && ntau == 2 && lp >= 16) {
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) part1[i][h] += a4[h];
          } else {
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) accv[i][h] += a4[h];
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kGdPass; ++i) {
      const int c = lane + 64 * i;
      if (c >= D) continue;
      if (VCH) {
#pragma unroll
        for (int u = 0; u < ntau; ++u) {
          const int tau = tau0 + u;
          if (tau * g >= r1) break;
          const size_t si = (bh * (size_t)(a.tcap / g) + tau) * D + c;
          const float sv = half_to_float(a.vs[si]), zv = half_to_float(a.vz[si]);
#pragma unroll
          for (int h = 0; h < kMaxG; ++h)
            o[i][h] += sv * ((u ? part1[i][h] : accv[i][h]) * kCodeScale) + zv * psum[u][h];
        }
      } else {
        const int j = c / g;
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) o[i][h] += accv[i][h] * kCodeScale + s_zs[wave][j][h];
      }
    }
    wave_lds_sync();  // the next block's weights overwrite this block's
  }

  // ---- combine the waves, write the range's partial
  __syncthreads();
  F4* s_o = reinterpret_cast<F4*>(s_buf);  // [wave][c], heads in F4
#pragma unroll
  for (int i = 0; i < kGdPass; ++i) {
    const int c = lane + 64 * i;
    if (c < D) {
      F4 f;
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) f.v[h] = o[i][h];
      s_o[wave * kGdMaxD + c] = f;
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      s_m[wave][h] = m[h];
      s_l[wave][h] = l[h];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kGdThreads) {
    const int h = idx / D, c = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kGdWaves; ++w) M = fmaxf(M, s_m[w][h]);
    const size_t row = (size_t)b * a.hq + h0 + h;
    float out = 0.f, lse = -INFINITY;
    if (M != -INFINITY) {
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < kGdWaves; ++w) {
        const float f = exp2f(s_m[w][h] - M);  // a wave with no token: m = -inf, f = 0
        num += f * s_o[w * kGdMaxD + c].v[h];
        den += f * s_l[w][h];
      }
      out = num / den;
      lse = (M + log2f(den)) * 0.69314718055994531f;
    }
    a.o_part[(row * S + s) * D + c] = out;
    if (c == 0) a.lse_part[row * S + s] = lse;
  }
}

// One work-group per query row: out = sum_s w_s O_s / sum_s w_s with
// w_s = e^(lse_s - max lse), lse = max + ln sum_s w_s; a row with no token
// gives out = 0 and lse = -inf.  The weights are computed once per row into
// LDS; each thread then sums its channels over the ranges.
__global__ __launch_bounds__(kGdThreads) void gd_merge(const GenericArgs a) {
  __shared__ float s_wt[kMaxSplits];
  __shared__ float s_red[2][kGdWaves];
  const size_t row = blockIdx.x;
  const int S = a.splits, D = a.d, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* lp = a.lse_part + row * S;
  float mx = -INFINITY;
  for (int s = tid; s < S; s += kGdThreads) mx = fmaxf(mx, lp[s]);
  mx = wave_max(mx);
  if (lane == 0) s_red[0][wave] = mx;
  __syncthreads();
  float M = s_red[0][0];
#pragma unroll
  for (int w = 1; w < kGdWaves; ++w) M = fmaxf(M, s_red[0][w]);
  float den = 0.f;
  for (int s = tid; s < S; s += kGdThreads) {
    const float w = M != -INFINITY ? expf(lp[s] - M) : 0.f;
    s_wt[s] = w;
    den += w;
  }
  den = wave_sum(den);
  if (lane == 0) s_red[1][wave] = den;
  __syncthreads();
  den = 0.f;
#pragma unroll
  for (int w = 0; w < kGdWaves; ++w) den += s_red[1][w];
  const float* op = a.o_part + row * S * (size_t)D;
  for (int c = tid; c < D; c += kGdThreads) {
    float num = 0.f;
#pragma unroll 8
    for (int s = 0; s < S; ++s) num += s_wt[s] * op[(size_t)s * D + c];  // empty ranges: weight 0, partial 0
    a.out[row * D + c] = float_to_bf16(M != -INFINITY ? num / den : 0.f);
  }
  if (tid == 0 && a.lse) a.lse[row] = M != -INFINITY ? M + logf(den) : -INFINITY;
}

template <int BITS, bool KCH, bool VCH>
const void* split_kernel(int group) {
  if (group == 32) return (const void*)gd_split<BITS, KCH, VCH, 32>;
  if (group == 64) return (const void*)gd_split<BITS, KCH, VCH, 64>;
  return (const void*)gd_split<BITS, KCH, VCH, 128>;
}

const void* pick(int bits, bool kch, bool vch, int group) {
  if (bits == 2) {
    if (kch) return vch ? split_kernel<2, true, true>(group) : split_kernel<2, true, false>(group);
    return vch ? split_kernel<2, false, true>(group) : split_kernel<2, false, false>(group);
  }
  if (kch) return vch ? split_kernel<4, true, true>(group) : split_kernel<4, true, false>(group);
  return vch ? split_kernel<4, false, true>(group) : split_kernel<4, false, false>(group);
}

size_t dyn_lds(bool kch, int d) { return kch ? (size_t)kGdWaves * 2 * d * sizeof(F4) : 0; }

}  // namespace

hipError_t generic_occupancy(int bits, bool kch, bool vch, int group, int d, int* per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, pick(bits, kch, vch, group), kGdThreads,
                                                      dyn_lds(kch, d));
}

hipError_t launch_decode_generic(int bits, bool kch, bool vch, const GenericArgs& a, hipStream_t stream,
                                 const LaunchEvents& ev) {
  hipError_t e = hipSuccess;
  if (ev.start) e = hipEventRecord(ev.start, stream);
  if (e != hipSuccess) return e;
  void* args[] = {(void*)&a};
  e = hipLaunchKernel(pick(bits, kch, vch, a.group), dim3(a.batch * a.pairs, a.splits), dim3(kGdThreads), args,
                     dyn_lds(kch, a.d), stream);
  if (e != hipSuccess) return e;
  e = hipLaunchKernel((const void*)gd_merge, dim3(a.batch * a.hq), dim3(kGdThreads), args, 0, stream);
  if (e != hipSuccess) return e;
  if (ev.stop) e = hipEventRecord(ev.stop, stream);
  return e;
}

}  // namespace foscar
