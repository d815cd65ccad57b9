// Split-KV decode attention over a 2-/4-bit quantised KV cache, gfx950.
//
// Method: FOSCAR ("Accelerating Decode Attention over 2- and 4-Bit KV Caches
// through Affine Folding", arXiv 2611.09722, abstract) as explained on
// "FOSCAR speeds up 2-bit KV decode -- Affine folding of KV dequantization"
// (learnaivisually): value = s*q + z per group (encoding paragraph); fold rule
// and fold-placement table: token-wise K and channel-wise V take acc-fold
// (scale the finished partial sum of a group once), channel-wise K and
// token-wise V take operand-fold (pre-scale Q or the softmax weights P); each
// offset becomes a correction z * (sum of the other operand); key-side
// corrections land before the softmax and value-side ones before the final
// division; an unscaled partial sum never crosses a group boundary.
//
// Work decomposition (MI355X-native; the pages' Hopper/Blackwell pipelines
// are not used):
//   * grid = (ranges S, KV heads, sequences); a work-group of 4 waves owns one
//     token range of one (sequence, KV head); waves take 64-token tiles (or
//     g-token units when a channel-wise group is longer than a tile) in turn;
//   * each wave streams its tiles HBM -> LDS with global_load_lds (dwordx4),
//     NS tiles deep in a per-wave ring, then reads lane l's data (token l's
//     packed key row, the value words of channels 2l, 2l+1, the quad's scales)
//     into registers; no registers are held by loads in flight;
//   * codes become matrix-core operands by one AND-OR per fp16 pair: a code
//     dropped into the mantissa under a fixed exponent reads as C + q (C a
//     power of two), and the C*sum(other operand) it adds is removed once per
//     row together with the offset correction -- no per-value convert or FMA;
//   * QK^T: v_mfma_f32_4x4x4_16b_f16, block = 4 tokens x 4 query heads, so
//     each lane ends with 4 dense scores (4 tokens of its quad, one query head)
//     and the key-side fold, mask and online softmax run on dense registers;
//   * P V: the same instruction with blocks over channels; the 4x4 P block of
//     every quad is shared through LDS (one 8-byte store, eight 16-byte loads
//     per lane per tile);
//   * online softmax with the exact running max of each query head (DPP,
//     ds_swizzle and ds_bpermute reductions across the 16 lanes of a head; the
//     accumulators are rescaled only when a max rises);
//   * a range's partial (O, lse) goes to a workspace with device-coherent (sc1)
//     relaxed stores; after its stores complete (vmcnt(0)) a work-group counts
//     its arrival on the pair's counter, and the last to arrive merges the
//     ranges by log-sum-exp, one memory round trip per 32 ranges: one decode
//     step is one kernel launch;
//   * a full-precision window of recent tokens is attended by extra work-groups
//     of the same launch (window_item) whose partials join that merge.
#include "decode_kernels.h"

namespace foscar {
namespace {

// One wave per query row: lane l rotates channels 2l, 2l + 1 (row r of dst = bf16(q_r H)).
__global__ __launch_bounds__(kWaves * 64) void rotate_query(const uint16_t* q, uint16_t* dst, int rows) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole waves
  const uint32_t w = reinterpret_cast<const uint32_t*>(q + (size_t)row * kHeadDim)[lane];
  reinterpret_cast<uint32_t*>(dst + (size_t)row * kHeadDim)[lane] = hadamard_bf16_pair(w, lane);
}

}  // namespace

hipError_t launch_rotate_query(int rows, const uint16_t* q, uint16_t* dst, hipStream_t stream, hipEvent_t start) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + kWaves - 1) / kWaves);
  if (start)
    hipExtLaunchKernelGGL(rotate_query, grid, dim3(kWaves * 64), 0, stream, start, nullptr, 0, q, dst, rows);
  else
    hipLaunchKernelGGL(rotate_query, grid, dim3(kWaves * 64), 0, stream, q, dst, rows);
  return hipGetLastError();
}

// the contiguous cache without rotation: instantiated here
hipError_t launch_split_plain(int bits, bool kch, bool vch, int group, int batch, int hkv, const SplitArgs& sa,
                              hipStream_t stream, int* per_cu, const LaunchEvents& ev) {
  return launch_variant<false, false>(bits, kch, vch, group, batch, hkv, sa, stream, per_cu, ev);
}

hipError_t launch_decode(int bits, bool k_channel, bool v_channel, int group, int batch, int hkv,
                         const SplitArgs& sa, hipStream_t stream, const LaunchEvents& ev) {
  const bool paged = sa.block_table != nullptr, rot = sa.rot != 0;
  auto* fn = paged ? (rot ? launch_split_paged_rot : launch_split_paged)
                   : (rot ? launch_split_rot : launch_split_plain);
  return fn(bits, k_channel, v_channel, group, batch, hkv, sa, stream, nullptr, ev);
}

hipError_t decode_occupancy(int bits, bool k_channel, bool v_channel, int group, bool paged, bool rot, int* per_cu) {
  SplitArgs sa{};
  const LaunchEvents none{};
  auto* fn = paged ? (rot ? launch_split_paged_rot : launch_split_paged)
                   : (rot ? launch_split_rot : launch_split_plain);
  return fn(bits, k_channel, v_channel, group, 0, 0, sa, nullptr, per_cu, none);
}

}  // namespace foscar
