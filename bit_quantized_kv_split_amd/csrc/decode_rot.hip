// Split decode over a rotated cache (keys and/or values stored as Hadamard-
// rotated rows): the instances of the decode kernels that take the cache's
// output back by H and give the full-precision window the caller's query
// (decode_kernels.h, ROT = true).  Kept apart from the unrotated instances,
// whose kernels carry none of this code.
#include "decode_kernels.h"

namespace foscar {

hipError_t launch_split_rot(int bits, bool kch, bool vch, int group, int batch, int hkv, const SplitArgs& sa,
                            hipStream_t stream, int* per_cu, const LaunchEvents& ev) {
  return launch_variant<false, true>(bits, kch, vch, group, batch, hkv, sa, stream, per_cu, ev);
}

}  // namespace foscar
