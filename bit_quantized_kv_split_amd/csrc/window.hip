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
// One work-group of 256 threads per (sequence, KV head):
//   * the G <= 4 query rows go to LDS as fp32;
//   * scores: thread t takes window tokens t, t + 256, ...: it reads the key
//     row once and forms the G dot products (bf16 x bf16 products are exact in
//     fp32) into an LDS score table;
//   * max and sum per query row by block reductions, weights p = exp(s - m)
//     in place;
//   * output: thread (i, j) accumulates query row i, channels 2j and 2j+1 over
//     the window, reading value rows as 256-byte coalesced lines.
#include <hip/hip_runtime.h>
#include <math.h>

#include "foscar_internal.h"

namespace foscar {
namespace {

constexpr int kWinThreads = 256;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(kWinThreads) void window_attend(const WindowArgs a) {
  constexpr int D = kHeadDim;
  const int b = blockIdx.y, h = blockIdx.x;
  const int G = a.g_heads;
  const int tid = threadIdx.x;
  const int W = min(max(a.wlens[b], 0), a.wcap);
  __shared__ float s_q[kMaxG][D];
  __shared__ float s_red[4];
  extern __shared__ float s_p[];  // [kMaxG][wcap] scores, then weights
  const size_t row0 = (size_t)b * a.hq + (size_t)h * G;
  for (int idx = tid; idx < kMaxG * D; idx += kWinThreads) {
    const int i = idx / D, c = idx % D;
    s_q[i][c] = (i < G) ? __uint_as_float((uint32_t)a.q[(row0 + i) * D + c] << 16) : 0.f;
  }
  __syncthreads();
  const size_t kv0 = ((size_t)b * a.hkv + h) * (size_t)a.wcap * D;
  const uint4* wk = reinterpret_cast<const uint4*>(a.wk + kv0);
  for (int t = tid; t < W; t += kWinThreads) {
    float acc[kMaxG] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int k = 0; k < D / 8; ++k) {
      const uint4 w = wk[(size_t)t * (D / 8) + k];
      const float x[8] = {bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y), bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w)};
#pragma unroll
      for (int i = 0; i < kMaxG; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i] = fmaf(s_q[i][8 * k + e], x[e], acc[i]);
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
    m[i] = block_max(v, s_red);
    float sum = 0.f;
    for (int t = tid; t < W; t += kWinThreads) {
      const float p = __expf(s_p[i * a.wcap + t] - m[i]);
      s_p[i * a.wcap + t] = p;
      sum += p;
    }
    l[i] = block_sum(sum, s_red);
  }
  __syncthreads();
  const int i = tid >> 6, j = tid & 63;  // query row i, channels 2j, 2j+1
  if (i >= G) return;
  const uint32_t* wv = reinterpret_cast<const uint32_t*>(a.wv + kv0) + j;
  float o0 = 0.f, o1 = 0.f;
  const float* p = s_p + i * a.wcap;
#pragma unroll 4
  for (int t = 0; t < W; ++t) {
    const uint32_t w = wv[(size_t)t * (D / 2)];
    o0 = fmaf(p[t], bf_lo(w), o0);
    o1 = fmaf(p[t], bf_hi(w), o1);
  }
  const size_t row = row0 + i;
  const float li = (i == 0) ? l[0] : (i == 1) ? l[1] : (i == 2) ? l[2] : l[3];
  const float mi = (i == 0) ? m[0] : (i == 1) ? m[1] : (i == 2) ? m[2] : m[3];
  const bool empty = W == 0;
  a.o[row * D + 2 * j] = empty ? 0.f : o0 / li;
  a.o[row * D + 2 * j + 1] = empty ? 0.f : o1 / li;
  if (j == 0) a.lse[row] = empty ? -INFINITY : mi + __logf(li);
}

}  // namespace

hipError_t launch_window(const WindowArgs& a, int batch, hipStream_t stream) {
  const size_t lds = sizeof(float) * kMaxG * (size_t)a.wcap;
  hipLaunchKernelGGL(window_attend, dim3(a.hkv, batch), dim3(kWinThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace foscar
