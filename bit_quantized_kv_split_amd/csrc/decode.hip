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
//   * grid = (work pairs, ranges S); a work pair is (sequence, KV head, group
//     of at most 4 of the KV head's query heads); a work-group of 4 waves owns
//     one token range of one pair; waves take 64-token tiles (or g-token units
//     when a channel-wise group is longer than a tile) in turn;
//   * each wave streams its tiles HBM -> LDS with buffer loads straight to LDS
//     (dwordx4) into a one-tile slot per wave, copies lane l's data into
//     registers and refills the slot with the next tile before working on the
//     copy; no registers are held by loads in flight;
//   * token-wise keys: QK^T on the block-scaled matrix cores
//     (v_mfma_scale_f32_16x16x128_f8f6f4): an INT2 code under one AND is an fp4
//     operand, an INT4 code an fp8 one, the query two exact e4m3 terms with one
//     E8M0 scale per row; a 64-token tile is 4 blocks of 16 tokens laid out so
//     that each lane ends with one query head's scores for the 4 tokens of a quad;
//   * channel-wise keys and every P V product: v_mfma_f32_4x4x4_16b_f16 with
//     code operands built by one AND-OR per fp16 pair (a code dropped into the
//     mantissa under a fixed exponent reads as C + q; the C * sum(other operand)
//     it adds is removed once per row) -- no per-value convert or FMA anywhere;
//   * online softmax with the exact running max of each query head (DPP and
//     permlane reductions; the accumulators are rescaled only when a max rises);
//   * a range's partial (O, lse) goes to a workspace with device-coherent (sc1)
//     relaxed stores; after its stores complete a work-group counts its arrival
//     on the pair's counter, and the last to arrive merges the ranges by
//     log-sum-exp, one memory round trip per 32 ranges: one decode step is one
//     kernel launch;
//   * a full-precision window of recent tokens is attended by extra work-groups
//     of the same launch (window_item) whose partials join that merge.
// The kernel templates are in decode_kernels.h.  This file instantiates the
// contiguous, unrotated variant and dispatches a call to one of the four
// variants (contiguous or paged, unrotated or rotated), each instantiated in a
// source file of its own.
#include "decode_kernels.h"

namespace foscar {

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

#ifdef FOSCAR_TIMELINE
// the timeline of the contiguous, unrotated instances (libfoscar_timeline.so only)
extern "C" int foscar_timeline_clear(void* stream) {  // asynchronous on `stream`: no gap before the next launch
  void* t = nullptr;
  hipError_t e = hipGetSymbolAddress(&t, HIP_SYMBOL(g_timeline));
  if (e == hipSuccess) e = hipMemsetAsync(t, 0, sizeof(g_timeline), (hipStream_t)stream);
  return (int)e;
}
extern "C" int foscar_timeline_read(void* host, int wgs) {  // host: u64 [wgs][8][8], wgs <= 8192
  if (wgs < 0 || wgs > kTimelineWgs) return -1;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_timeline), (size_t)wgs * kTimelineItems * 8 * 8, 0,
                                  hipMemcpyDeviceToHost);
}
#endif

hipError_t decode_occupancy(int bits, bool k_channel, bool v_channel, int group, bool paged, bool rot, int* per_cu) {
  SplitArgs sa{};
  const LaunchEvents none{};
  auto* fn = paged ? (rot ? launch_split_paged_rot : launch_split_paged)
                   : (rot ? launch_split_rot : launch_split_plain);
  return fn(bits, k_channel, v_channel, group, 0, 0, sa, nullptr, per_cu, none);
}

}  // namespace foscar
