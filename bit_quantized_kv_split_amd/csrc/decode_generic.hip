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
// words; the query operand is an LDS broadcast), the online softmax reduces
// over the wave, and the weighted values have lane = channel (64 consecutive
// channels per pass, so each value-word load is one coalesced row segment).
// Every step runs on the vector ALUs: at these head dimensions a 64-token
// block is too small a contraction per wave for the matrix cores to repay the
// operand shuffles.  Tokens at or past the sequence length are never loaded.
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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
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

template <int BITS, bool KCH, bool VCH>
__global__ __launch_bounds__(kGdThreads) void gd_split(const GenericArgs a) {
  constexpr int E = 32 / BITS;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const int D = a.d, g = a.group, G = a.g_heads, S = a.splits;
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
  __shared__ float s_qsum[kGdMaxD / 32][kMaxG];                 // token-wise K: sum of q over channel group j
  __shared__ F4 s_qt[KCH ? kGdWaves * 2 * kGdMaxD : 1];        // channel-wise K: q~ of a block's (<= 2) token groups
  __shared__ float s_bias[kGdWaves][2][kMaxG];                  // channel-wise K: sum_c q z of those groups
  constexpr int kWSize = VCH ? kGdWaves * 64 : kGdWaves * (kGdMaxD / 32) * 64;
  constexpr int kOSize = kGdWaves * kGdMaxD;                     // combine: o[w][c] (heads in F4)
  __shared__ F4 s_w[kWSize > kOSize ? kWSize : kOSize];         // weights of a block; after the loop, the combine
  __shared__ float s_zs[kGdWaves][kGdMaxD / 32][kMaxG];         // token-wise V: sum_t p z per channel group
  __shared__ float s_m[kGdWaves][kMaxG], s_l[kGdWaves][kMaxG];

  for (int i = tid; i < D; i += kGdThreads) {
    F4 f;
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) f.v[h] = h < G ? bf16_to_float(a.q[((size_t)b * a.hq + h0 + h) * D + i]) : 0.f;
    s_q[i] = f;
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
    const int ntau = (KCH || VCH) && g < 64 ? 2 : 1;  // token groups a 64-token block meets (blocks start at multiples of 64)

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
            s_qt[(wave * 2 + u) * kGdMaxD + c] = qt;
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
        const F4* qt = s_qt + (wave * 2 + u) * kGdMaxD;
        for (int w = 0; w < W; ++w) {
          const uint32_t word = krow[w];
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float cf = (float)((word >> elem_shift(BITS, e)) & MASK);
            const F4 qv = qt[w * E + e];
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) sc[h] = __builtin_fmaf(qv.v[h], cf, sc[h]);
          }
        }
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) sc[h] += s_bias[wave][u][h];
      } else {
        const int wpg = g / E;  // words of a channel group
        for (int j = 0; j < NJ; ++j) {
          float acc[kMaxG];
#pragma unroll
          for (int h = 0; h < kMaxG; ++h) acc[h] = 0.f;
          for (int w = j * wpg; w < j * wpg + wpg; ++w) {
            const uint32_t word = krow[w];
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const float cf = (float)((word >> elem_shift(BITS, e)) & MASK);
              const F4 qv = s_q[w * E + e];
#pragma unroll
              for (int h = 0; h < kMaxG; ++h) acc[h] = __builtin_fmaf(qv.v[h], cf, acc[h]);
            }
          }
          const size_t si = (bh * a.tcap + t) * (size_t)NJ + j;
          const float sk = half_to_float(a.ks[si]), zk = half_to_float(a.kz[si]);
#pragma unroll
          for (int h = 0; h < kMaxG; ++h) sc[h] += sk * acc[h] + zk * s_qsum[j][h];
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
      F4 pw;
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) pw.v[h] = p[h];
      s_w[wave * 64 + lane] = pw;
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
        F4 pw;
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
          pw.v[h] = p[h] * sv;
          const float zs = wave_sum(p[h] * zv);
          if (lane == 0) s_zs[wave][j][h] = zs;
        }
        s_w[(wave * (kGdMaxD / 32) + j) * 64 + lane] = pw;
      }
    }
    wave_lds_sync();

    // ---- weighted values, lane = channel
    const int tw0 = blk / E, tw1 = min(blk + 64, r1);  // word rows tw0 .. while tw * E < tw1
#pragma unroll
    for (int i = 0; i < kGdPass; ++i) {
      const int c = lane + 64 * i;
      if (c >= D) break;
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) o[i][h] *= alpha[h];
      float part[2][kMaxG];
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) part[0][h] = part[1][h] = 0.f;
      const int j = c / g;
      for (int tw = tw0; tw * E < tw1; ++tw) {
        const uint32_t word = a.pv[(bh * (size_t)(a.tcap / E) + tw) * D + c];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int local = tw * E + e - blk;  // 0 .. 63; weights past the length are zero
          const float cf = (float)((word >> elem_shift(BITS, e)) & MASK);
          if (VCH) {
            const F4 pw = s_w[wave * 64 + local];
            const int u = local >> 5;
            if (ntau == 2 && u == 1) {
#pragma unroll
              for (int h = 0; h < kMaxG; ++h) part[1][h] = __builtin_fmaf(pw.v[h], cf, part[1][h]);
            } else {
#pragma unroll
              for (int h = 0; h < kMaxG; ++h) part[0][h] = __builtin_fmaf(pw.v[h], cf, part[0][h]);
            }
          } else {
            const F4 pw = s_w[(wave * (kGdMaxD / 32) + j) * 64 + local];
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) o[i][h] = __builtin_fmaf(pw.v[h], cf, o[i][h]);
          }
        }
      }
      if (VCH) {
        for (int u = 0; u < ntau; ++u) {
          const int tau = tau0 + u;
          if (tau * g >= r1) break;
          const size_t si = (bh * (size_t)(a.tcap / g) + tau) * D + c;
          const float sv = half_to_float(a.vs[si]), zv = half_to_float(a.vz[si]);
#pragma unroll
          for (int h = 0; h < kMaxG; ++h) o[i][h] += sv * part[u][h] + zv * psum[u][h];
        }
      } else {
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) o[i][h] += s_zs[wave][j][h];
      }
    }
    wave_lds_sync();  // the next block's weights overwrite this block's
  }

  // ---- combine the waves, write the range's partial
  __syncthreads();
  F4* s_o = s_w;  // [wave][c], heads in F4
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
// gives out = 0 and lse = -inf.
__global__ __launch_bounds__(kGdThreads) void gd_merge(const GenericArgs a) {
  const size_t row = blockIdx.x;
  const int S = a.splits, D = a.d;
  const float* lp = a.lse_part + row * S;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, lp[s]);
  float den = 0.f;
  if (M != -INFINITY)
    for (int s = 0; s < S; ++s) den += expf(lp[s] - M);
  for (int c = threadIdx.x; c < D; c += kGdThreads) {
    float num = 0.f;
    if (M != -INFINITY)
      for (int s = 0; s < S; ++s) {
        const float w = expf(lp[s] - M);
        if (w != 0.f) num += w * a.o_part[(row * S + s) * D + c];
      }
    a.out[row * D + c] = float_to_bf16(M != -INFINITY ? num / den : 0.f);
  }
  if (threadIdx.x == 0 && a.lse) a.lse[row] = M != -INFINITY ? M + logf(den) : -INFINITY;
}

template <int BITS, bool KCH, bool VCH>
const void* split_kernel() {
  return (const void*)gd_split<BITS, KCH, VCH>;
}

const void* pick(int bits, bool kch, bool vch) {
  if (bits == 2) {
    if (kch) return vch ? split_kernel<2, true, true>() : split_kernel<2, true, false>();
    return vch ? split_kernel<2, false, true>() : split_kernel<2, false, false>();
  }
  if (kch) return vch ? split_kernel<4, true, true>() : split_kernel<4, true, false>();
  return vch ? split_kernel<4, false, true>() : split_kernel<4, false, false>();
}

}  // namespace

hipError_t generic_occupancy(int bits, bool kch, bool vch, int* per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, pick(bits, kch, vch), kGdThreads, 0);
}

hipError_t launch_decode_generic(int bits, bool kch, bool vch, const GenericArgs& a, hipStream_t stream,
                                 const LaunchEvents& ev) {
  hipError_t e = hipSuccess;
  if (ev.start) e = hipEventRecord(ev.start, stream);
  if (e != hipSuccess) return e;
  void* args[] = {(void*)&a};
  e = hipLaunchKernel(pick(bits, kch, vch), dim3(a.batch * a.pairs, a.splits), dim3(kGdThreads), args, 0, stream);
  if (e != hipSuccess) return e;
  e = hipLaunchKernel((const void*)gd_merge, dim3(a.batch * a.hq), dim3(kGdThreads), args, 0, stream);
  if (e != hipSuccess) return e;
  if (ev.stop) e = hipEventRecord(ev.stop, stream);
  return e;
}

}  // namespace foscar
