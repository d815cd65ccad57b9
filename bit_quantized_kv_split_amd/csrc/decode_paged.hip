// Split decode over a paged cache: the instances of the decode kernels whose
// tiles reach the cache through a block table (decode_kernels.h, PAGED = true).
#include "decode_kernels.h"

namespace foscar {
namespace {

template <int BITS, bool KCH, bool VCH>
hipError_t launch_g(int group, int batch, int hkv, const SplitArgs& sa, hipStream_t stream, int* per_cu,
                    const LaunchEvents& ev) {
  return launch_gp<BITS, KCH, VCH, true>(group, batch, hkv, sa, stream, per_cu, ev);
}

template <int BITS>
hipError_t launch_bits(bool kch, bool vch, int group, int batch, int hkv, const SplitArgs& sa, hipStream_t stream,
                       int* per_cu, const LaunchEvents& ev) {
  if (kch) {
    return vch ? launch_g<BITS, true, true>(group, batch, hkv, sa, stream, per_cu, ev)
               : launch_g<BITS, true, false>(group, batch, hkv, sa, stream, per_cu, ev);
  }
  return vch ? launch_g<BITS, false, true>(group, batch, hkv, sa, stream, per_cu, ev)
             : launch_g<BITS, false, false>(group, batch, hkv, sa, stream, per_cu, ev);
}

}  // namespace

hipError_t launch_decode_paged(int bits, bool k_channel, bool v_channel, int group, int batch, int hkv,
                               const SplitArgs& sa, hipStream_t stream, const LaunchEvents& ev) {
  if (bits == 2) return launch_bits<2>(k_channel, v_channel, group, batch, hkv, sa, stream, nullptr, ev);
  return launch_bits<4>(k_channel, v_channel, group, batch, hkv, sa, stream, nullptr, ev);
}

hipError_t decode_occupancy_paged(int bits, bool k_channel, bool v_channel, int group, int* per_cu) {
  SplitArgs sa{};
  const LaunchEvents none{};
  if (bits == 2) return launch_bits<2>(k_channel, v_channel, group, 0, 0, sa, nullptr, per_cu, none);
  return launch_bits<4>(k_channel, v_channel, group, 0, 0, sa, nullptr, per_cu, none);
}

}  // namespace foscar
