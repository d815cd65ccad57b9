// Split decode over a paged cache: the instances of the decode kernels whose
// tiles reach the cache through a block table (decode_kernels.h, PAGED = true).
#include "decode_kernels.h"

namespace foscar {

hipError_t launch_split_paged(int bits, bool kch, bool vch, int group, int batch, int hkv, const SplitArgs& sa,
                              hipStream_t stream, int* per_cu, const LaunchEvents& ev) {
  return launch_variant<true, false>(bits, kch, vch, group, batch, hkv, sa, stream, per_cu, ev);
}

}  // namespace foscar
