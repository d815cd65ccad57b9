// Internal declarations shared by the host interface and the kernels of
// libfoscar (decode attention over a 2-/4-bit quantised KV cache, gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace foscar {

constexpr int kHeadDim = 128;   // D
constexpr int kTile = 64;       // tokens per wave tile (16 quads of 4)
constexpr int kWaves = 4;       // waves per work-group
constexpr int kMaxG = 4;        // query heads of one work pair (a wave's query rows)
constexpr int kMaxGqa = 16;     // query heads per KV head the interface takes (served as groups of <= kMaxG)
constexpr int kMapMaxB = 1024;   // largest batch the device-side work order handles (64 lanes x 16)
constexpr int kMaxSplits = 512;  // ranges per sequence (bounds the workspace and the merge passes)

// Arguments of the decode kernel (one work-group per (range, KV head, sequence)).
// The last work-group to finish the ranges of a (sequence, KV head) merges them.
struct SplitArgs {
  const uint16_t* q;         // bf16 [B][Hq][D] the caller's query (rotated keys: each work-group rotates its rows)
  const uint32_t* pk;        // [B][Hkv][Tcap][D*bits/32]
  const uint32_t* pv;        // [B][Hkv][Tcap*bits/32][D]
  const uint16_t* ks;        // fp16 key scales   (token-wise [B][Hkv][Tcap][D/g], channel-wise [B][Hkv][Tcap/g][D])
  const uint16_t* kz;        // fp16 key offsets
  const uint16_t* vs;        // fp16 value scales
  const uint16_t* vz;        // fp16 value offsets
  const int32_t* seq_lens;   // [B]
  uint16_t* out;             // bf16 [B][Hq][D]
  float* lse;                // fp32 [B][Hq] or null
  float* o_part;             // fp32 [B][Hq][S][D]   normalised partial output of each range
  float* lse_part;           // fp32 [B][Hq][S]      natural-log lse of each range
  int32_t* counters;         // [B][pairs] ranges finished; zero between calls
  // Hq; work pairs per sequence (Hkv * kv_group); query heads per pair (Hq / Hkv / kv_group);
  // pairs per KV head: pair h of a sequence reads KV head h / kv_group
  int32_t hq, hkv, g_heads, kv_group;
  int32_t tcap;              // Tcap
  int32_t splits;            // S
  int32_t chunk;             // tokens per range (multiple of the wave unit)
  float sm_log2;             // sm_scale * log2(e)
  int32_t persistent;        // 1: grid_wgs work-groups take work items from work_ctr (see split_decode)
  int32_t grid_wgs;          // persistent grid size (one round of resident work-groups)
  int32_t batch;             // B
  // rotated cache (H: orthonormal Sylvester-Hadamard of order 128), bit 0: the cache keys are rows
  // of K H, and each work-group meets them with its query rows rotated (bf16(q H)); bit 1: the
  // cache values are rows of V H, and the cache's weighted value sum is taken back by H before the
  // window's terms join it.
  int32_t rot;
  int32_t* work_ctr;         // [2] items taken, work-groups left; zero between calls
  // paged cache (block_table != null): pk .. vz are pools of num_blocks blocks of block_size
  // tokens, [num_blocks][Hkv][block_size][..] in the layouts above with Tcap = block_size, and
  // logical block j of sequence b (tokens j * block_size ..) is pool block block_table[b][j]
  const int32_t* block_table;  // [B][Tcap / block_size]
  int32_t block_size;          // multiple of 64 (and of g for a channel-wise side)
  int32_t num_blocks;
  float* win_o;              // fp32 [B][Hq][win_wgs][D] normalised outputs over a full-precision window, or null
  float* win_lse;            // fp32 [B][Hq][win_wgs] their natural-log lse (-inf: no window token)
  // window attended inside this launch (win_wgs = 0: no window): win_wgs more work-groups per pair
  // (grid rows 0 .. win_wgs-1 with the ranges in the rows after them, or the first B * Hkv * win_wgs
  // blocks of a persistent grid), work-group j taking window tokens [j * win_chunk, +win_chunk); each
  // row gets win_wgs window partials
  int32_t win_wgs;
  int32_t win_chunk;         // <= kFusedWindowMax
  const uint16_t* win_k;     // bf16 [B][Hkv][win_cap][D]
  const uint16_t* win_v;
  const int32_t* win_lens;   // [B]
  int32_t win_cap;
  float win_sm;              // softmax scale (natural units)
};
constexpr int kMaxWindowWgs = 8;      // window work-groups per pair inside the decode launch
constexpr int kFusedWindowMax = 512;  // window tokens of one work-group inside the decode launch
constexpr int kMaxWindow = kMaxWindowWgs * kFusedWindowMax;  // tokens of a window: 4096

// Events the dispatch records around the kernel (either may be null).
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
hipError_t launch_decode(int bits, bool k_channel, bool v_channel, int group, int batch, int hkv,
                         const SplitArgs& sa, hipStream_t stream, const LaunchEvents& ev);  // by sa.block_table, sa.rot

// Work-groups of the decode kernel for (bits, layout sides, group, paged, rotated) one CU holds at once.
hipError_t decode_occupancy(int bits, bool k_channel, bool v_channel, int group, bool paged, bool rot, int* per_cu);
// The four variants of the decode kernel, each instantiated in a source file of its own (decode.hip,
// decode_paged.hip, decode_rot.hip, decode_paged_rot.hip): launch, or report the occupancy in *per_cu.
using SplitLauncher = hipError_t (*)(int bits, bool kch, bool vch, int group, int batch, int hkv,
                                     const SplitArgs& sa, hipStream_t stream, int* per_cu, const LaunchEvents& ev);
hipError_t launch_split_plain(int bits, bool kch, bool vch, int group, int batch, int hkv, const SplitArgs& sa,
                              hipStream_t stream, int* per_cu, const LaunchEvents& ev);
hipError_t launch_split_paged(int bits, bool kch, bool vch, int group, int batch, int hkv, const SplitArgs& sa,
                              hipStream_t stream, int* per_cu, const LaunchEvents& ev);
hipError_t launch_split_rot(int bits, bool kch, bool vch, int group, int batch, int hkv, const SplitArgs& sa,
                            hipStream_t stream, int* per_cu, const LaunchEvents& ev);
hipError_t launch_split_paged_rot(int bits, bool kch, bool vch, int group, int batch, int hkv, const SplitArgs& sa,
                                  hipStream_t stream, int* per_cu, const LaunchEvents& ev);
// Decode for head dimensions other than kHeadDim (decode_generic.hip): a multiple of 32 up to
// kGdMaxD, plain caches (no window, paging or rotation).  One work-group per (work pair, range)
// writes the range's partial; a second launch merges the ranges of each query row.
constexpr int kGdMaxD = 256;
struct GenericArgs {
  const uint16_t* q;          // bf16 [B][Hq][D]
  const uint32_t* pk;         // [B][Hkv][Tcap][D*bits/32]
  const uint32_t* pv;         // [B][Hkv][Tcap*bits/32][D]
  const uint16_t* ks;         // fp16 scales / offsets in the layouts of SplitArgs
  const uint16_t* kz;
  const uint16_t* vs;
  const uint16_t* vz;
  const int32_t* seq_lens;    // [B]
  uint16_t* out;              // bf16 [B][Hq][D]
  float* lse;                 // fp32 [B][Hq] or null
  float* o_part;              // fp32 [B][Hq][S][D]
  float* lse_part;            // fp32 [B][Hq][S]
  // B; Hq; Hkv; work pairs per sequence (Hkv * kv_group); pairs per KV head; query heads per pair
  int32_t batch, hq, hkv, pairs, kv_group, g_heads;
  int32_t d;                  // D
  int32_t tcap;               // Tcap
  int32_t group;              // g
  int32_t splits;             // S
  int32_t chunk;              // tokens per range (a multiple of 64, and of g for a channel-wise side)
  float sm_log2;              // sm_scale * log2(e)
};
hipError_t launch_decode_generic(int bits, bool k_channel, bool v_channel, const GenericArgs& a, hipStream_t stream,
                                 const LaunchEvents& ev);
hipError_t generic_occupancy(int bits, bool k_channel, bool v_channel, int group, int d, int* per_cu);

// Quantise tokens [start_b, start_b + count_b) of new keys / values into the cache (quant.hip);
// rot bit 0 / bit 1: rotate the key / value rows by the orthonormal Hadamard matrix first.
hipError_t launch_quantize(int bits, bool k_channel, bool v_channel, int group, int rot, int batch, int hkv, int tcap,
                           int n_src, const void* k_src, const void* v_src, const int32_t* start, const int32_t* count,
                           void* pk, void* pv, void* ks, void* kz, void* vs, void* vz, hipStream_t stream);
hipError_t launch_pack(int bits, int side, int batch, int hkv, int tcap, int d, const uint8_t* codes, uint32_t* packed,
                       hipStream_t stream);
hipError_t launch_unpack(int bits, int side, int batch, int hkv, int tcap, int d, const uint32_t* packed,
                         uint8_t* codes, hipStream_t stream);

}  // namespace foscar
