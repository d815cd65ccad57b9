// Packing of logical codes into the packed word layout of the interface, and
// back.  E = 32/bits codes per word along the packed axis (channels for keys,
// tokens for values); element e of a word sits at bit bits*(e/2) + 16*(e%2),
// so that one AND-OR of a word yields two adjacent elements as an fp16 pair.
#include "foscar_internal.h"

namespace foscar {
namespace {

__device__ __forceinline__ int elem_shift(int bits, int e) { return bits * (e >> 1) + 16 * (e & 1); }

// keys: word i of the flat [B*Hkv*Tcap][D/E] array covers flat codes [i*E, i*E + E)
__global__ void pack_keys(int bits, const uint8_t* __restrict__ codes, uint32_t* __restrict__ packed, size_t nwords) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i >= nwords) return;
  const int E = 32 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  const uint8_t* c = codes + i * E;
  uint32_t w = 0;
  for (int e = 0; e < E; ++e) w |= ((uint32_t)c[e] & mask) << elem_shift(bits, e);
  packed[i] = w;
}

__global__ void unpack_keys(int bits, const uint32_t* __restrict__ packed, uint8_t* __restrict__ codes, size_t nwords) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i >= nwords) return;
  const int E = 32 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  const uint32_t w = packed[i];
  for (int e = 0; e < E; ++e) codes[i * E + e] = (uint8_t)((w >> elem_shift(bits, e)) & mask);
}

// values: word [bh][tw][c] covers codes [bh][tw*E + e][c], e < E
__global__ void pack_values(int bits, int tcap, int d, const uint8_t* __restrict__ codes,
                            uint32_t* __restrict__ packed, size_t nwords) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i >= nwords) return;
  const int E = 32 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  const int c = (int)(i % d);
  const size_t rest = i / d;
  const size_t tw = rest % (size_t)(tcap / E);
  const size_t bh = rest / (size_t)(tcap / E);
  const uint8_t* src = codes + (bh * tcap + tw * E) * d + c;
  uint32_t w = 0;
  for (int e = 0; e < E; ++e) w |= ((uint32_t)src[(size_t)e * d] & mask) << elem_shift(bits, e);
  packed[i] = w;
}

__global__ void unpack_values(int bits, int tcap, int d, const uint32_t* __restrict__ packed,
                              uint8_t* __restrict__ codes, size_t nwords) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i >= nwords) return;
  const int E = 32 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  const int c = (int)(i % d);
  const size_t rest = i / d;
  const size_t tw = rest % (size_t)(tcap / E);
  const size_t bh = rest / (size_t)(tcap / E);
  uint8_t* dst = codes + (bh * tcap + tw * E) * d + c;
  const uint32_t w = packed[i];
  for (int e = 0; e < E; ++e) dst[(size_t)e * d] = (uint8_t)((w >> elem_shift(bits, e)) & mask);
}

}  // namespace

hipError_t launch_pack(int bits, int side, int batch, int hkv, int tcap, int d, const uint8_t* codes, uint32_t* packed,
                       hipStream_t stream) {
  const size_t nwords = (size_t)batch * hkv * tcap * d * bits / 32;
  if (nwords == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((nwords + 255) / 256);
  if (side == 0)
    hipLaunchKernelGGL(pack_keys, dim3(blocks), dim3(256), 0, stream, bits, codes, packed, nwords);
  else
    hipLaunchKernelGGL(pack_values, dim3(blocks), dim3(256), 0, stream, bits, tcap, d, codes, packed, nwords);
  return hipGetLastError();
}

hipError_t launch_unpack(int bits, int side, int batch, int hkv, int tcap, int d, const uint32_t* packed,
                         uint8_t* codes, hipStream_t stream) {
  const size_t nwords = (size_t)batch * hkv * tcap * d * bits / 32;
  if (nwords == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((nwords + 255) / 256);
  if (side == 0)
    hipLaunchKernelGGL(unpack_keys, dim3(blocks), dim3(256), 0, stream, bits, packed, codes, nwords);
  else
    hipLaunchKernelGGL(unpack_values, dim3(blocks), dim3(256), 0, stream, bits, tcap, d, packed, codes, nwords);
  return hipGetLastError();
}

}  // namespace foscar
