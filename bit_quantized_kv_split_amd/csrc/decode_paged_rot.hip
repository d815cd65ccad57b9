// Split decode over a paged, rotated cache (decode_kernels.h, PAGED = true,
// ROT = true).
#include "decode_kernels.h"

namespace foscar {

hipError_t launch_split_paged_rot(int bits, bool kch, bool vch, int group, int batch, int hkv, const SplitArgs& sa,
                                  hipStream_t stream, int* per_cu, const LaunchEvents& ev) {
  return launch_variant<true, true>(bits, kch, vch, group, batch, hkv, sa, stream, per_cu, ev);
}

}  // namespace foscar
