// Attention of the decode query over a full-precision (bf16) window of recent
// tokens kept beside the quantised cache, gfx950.
//
// The FOSCAR explainer ("FOSCAR speeds up 2-bit KV decode -- Affine folding of
// KV dequantization", learnaivisually, accuracy paragraph) names
// full-precision windows of recent tokens as part of the accuracy recipe a
// 2-bit cache needs.  The window's tokens are extra keys and values of the
// same softmax: this kernel writes the window's normalised partial output and
// its log-sum-exp, and the decode kernel merges that partial with the cache's
// ranges by log-sum-exp, exactly as it merges two ranges of the cache.
//
// One work-group of 16 waves per (sequence, KV head); wave w takes the
// contiguous chunk w of the window's tokens:
//   * the G <= 4 query rows go to LDS as fp32;
//   * scores: lane l of wave w takes token (chunk start + l + 64k): one key
//     row read and the G dot products (bf16 x bf16 products are exact in
//     fp32; the query is broadcast from LDS 16 bytes at a time) into an LDS
//     score table;
//   * max and sum per query row over the 16 waves, weights p = exp(s - m) in
//     place;
//   * output: lane j of wave w accumulates channels 2j, 2j+1 of all G query
//     rows over the chunk's tokens (one 256-byte value row per wave and token,
//     16 rows in flight), then the 16 waves' sums are added through LDS.
#include <hip/hip_runtime.h>
#include <math.h>

#include "foscar_internal.h"

namespace foscar {
namespace {

constexpr int kWinWaves = 16;
constexpr int kWinThreads = 64 * kWinWaves;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// max / sum of v over the work-group, every thread gets the result (red: kWinWaves floats)
template <bool MAX>
__device__ __forceinline__ float block_reduce(float v, float* red) {
  for (int m = 32; m >= 1; m >>= 1) {
    const float o = __shfl_xor(v, m);
    v = MAX ? fmaxf(v, o) : v + o;
  }
  __syncthreads();  // red is free
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kWinWaves; ++w) r = MAX ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

__global__ __launch_bounds__(kWinThreads) void window_attend(const WindowArgs a) {
  constexpr int D = kHeadDim;
  const int b = blockIdx.y, h = blockIdx.x;
  const int G = a.g_heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int W = min(max(a.wlens[b], 0), a.wcap);
  const int chunk = (W + kWinWaves - 1) / kWinWaves;
  const int t0 = wave * chunk, t1 = min(t0 + chunk, W);
  __shared__ __align__(16) float s_q[kMaxG][D];
  __shared__ float s_red[kWinWaves];
  extern __shared__ __align__(16) float s_dyn[];  // [kMaxG][wcap] scores then weights; then [kWinWaves][kMaxG][D]
  float* s_p = s_dyn;
  float* s_o = s_dyn + kMaxG * a.wcap;
  const size_t row0 = (size_t)b * a.hq + (size_t)h * G;
  for (int idx = tid; idx < kMaxG * D; idx += kWinThreads) {
    const int i = idx / D, c = idx % D;
    s_q[i][c] = (i < G) ? __uint_as_float((uint32_t)a.q[(row0 + i) * D + c] << 16) : 0.f;
  }
  __syncthreads();
  const size_t kv0 = ((size_t)b * a.hkv + h) * (size_t)a.wcap * D;
  const uint4* wk = reinterpret_cast<const uint4*>(a.wk + kv0);
  for (int t = t0 + lane; t < t1; t += 64) {
    float acc[kMaxG] = {0.f, 0.f, 0.f, 0.f};
    const uint4* kr = wk + (size_t)t * (D / 8);
#pragma unroll 4
    for (int k = 0; k < D / 8; ++k) {
      const uint4 w = kr[k];
      const float x[8] = {bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y), bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w)};
#pragma unroll
      for (int i = 0; i < kMaxG; ++i) {
        const float4 qa = *reinterpret_cast<const float4*>(&s_q[i][8 * k]);
        const float4 qb = *reinterpret_cast<const float4*>(&s_q[i][8 * k + 4]);
        acc[i] = fmaf(qa.x, x[0], acc[i]);
        acc[i] = fmaf(qa.y, x[1], acc[i]);
        acc[i] = fmaf(qa.z, x[2], acc[i]);
        acc[i] = fmaf(qa.w, x[3], acc[i]);
        acc[i] = fmaf(qb.x, x[4], acc[i]);
        acc[i] = fmaf(qb.y, x[5], acc[i]);
        acc[i] = fmaf(qb.z, x[6], acc[i]);
        acc[i] = fmaf(qb.w, x[7], acc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kMaxG; ++i) s_p[i * a.wcap + t] = acc[i] * a.sm;
  }
  __syncthreads();
  float m[kMaxG], l[kMaxG];
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    float v = -INFINITY;
    for (int t = tid; t < W; t += kWinThreads) v = fmaxf(v, s_p[i * a.wcap + t]);
    m[i] = block_reduce<true>(v, s_red);
    float sum = 0.f;
    for (int t = tid; t < W; t += kWinThreads) {
      const float p = __expf(s_p[i * a.wcap + t] - m[i]);
      s_p[i * a.wcap + t] = p;
      sum += p;
    }
    l[i] = block_reduce<false>(sum, s_red);
  }
  __syncthreads();  // every weight is in place
  // weighted values of this wave's chunk: lane = channels 2 lane, 2 lane + 1, all query rows
  const uint32_t* wv = reinterpret_cast<const uint32_t*>(a.wv + kv0) + lane;
  float o[kMaxG][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
  for (int tb = t0; tb < t1; tb += 16) {
    uint32_t vr[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) vr[u] = (tb + u < t1) ? wv[(size_t)(tb + u) * (D / 2)] : 0u;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (tb + u >= t1) break;
      const float v0 = bf_lo(vr[u]), v1 = bf_hi(vr[u]);
#pragma unroll
      for (int i = 0; i < kMaxG; ++i) {
        const float p = s_p[i * a.wcap + tb + u];
        o[i][0] = fmaf(p, v0, o[i][0]);
        o[i][1] = fmaf(p, v1, o[i][1]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    s_o[(wave * kMaxG + i) * D + 2 * lane] = o[i][0];
    s_o[(wave * kMaxG + i) * D + 2 * lane + 1] = o[i][1];
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kWinThreads) {
    const int i = idx / D, c = idx % D;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWinWaves; ++w) sum += s_o[(w * kMaxG + i) * D + c];
    const float li = (i == 0) ? l[0] : (i == 1) ? l[1] : (i == 2) ? l[2] : l[3];
    const float mi = (i == 0) ? m[0] : (i == 1) ? m[1] : (i == 2) ? m[2] : m[3];
    const size_t row = row0 + i;
    a.o[row * D + c] = (W == 0) ? 0.f : sum / li;
    if (c == 0) a.lse[row] = (W == 0) ? -INFINITY : mi + __logf(li);
  }
}

}  // namespace

hipError_t launch_window(const WindowArgs& a, int batch, hipStream_t stream) {
  const size_t lds = sizeof(float) * kMaxG * ((size_t)a.wcap + (size_t)kWinWaves * kHeadDim);
  hipLaunchKernelGGL(window_attend, dim3(a.hkv, batch), dim3(kWinThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace foscar
