// Host side of libfoscar: the C interface declared in include/foscar.h.
// Every argument is checked before the first HIP call; errors are returned as
// codes, never thrown.  The only memory the library owns is the grow-only
// split workspace, one per (device, stream).
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <algorithm>
#include <mutex>
#include <utility>

#include "../../include/foscar.h"
#include "foscar_internal.h"

namespace {

thread_local int g_last_hip_error = 0;
thread_local foscar::LaunchEvents g_next_events;  // armed by foscar_record_next_launch

// [counters: counter_bytes][partials: bytes - counter_bytes].  The counter
// region keeps its place and size until the buffer grows, and holds nothing
// but counters, so counters that every call leaves at zero stay zero.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
  size_t counter_bytes = 0;
};

std::mutex g_ws_mutex;
std::map<std::pair<int, void*>, Workspace> g_ws;  // (device, stream) -> workspace
std::map<int, int> g_cus;                           // device -> compute units
std::map<long long, int> g_occ;                     // (device, bits, layout, group) -> resident work-groups per CU

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) ? FOSCAR_ENOMEM : FOSCAR_EHIP;
}

bool valid_group(int g) { return g == 32 || g == 64 || g == 128; }

// The kernels move packed words, scales and bf16 rows 16 bytes at a time and
// read the query, lengths and outputs 4 bytes at a time.
bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

// Shape checks shared by every entry point that takes dims.
int check_dims(const foscar_dims* d, bool need_heads_ratio) {
  if (!d) return FOSCAR_EINVAL;
  if (d->batch < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->head_dim < 1 || d->max_seq_len < 0)
    return FOSCAR_EINVAL;
  // 128 on every entry point; other multiples of 32 up to kGdMaxD: plain decode, pack and sizes
  if (d->head_dim != foscar::kHeadDim && (d->head_dim % 32 != 0 || d->head_dim > foscar::kGdMaxD))
    return FOSCAR_EUNSUPPORTED;
  if (need_heads_ratio) {
    if (d->num_q_heads % d->num_kv_heads != 0) return FOSCAR_EINVAL;
    if (d->num_q_heads / d->num_kv_heads > foscar::kMaxGqa) return FOSCAR_EUNSUPPORTED;
  }
  return FOSCAR_OK;
}

// The kernels serve one work pair of at most kMaxG query heads (a wave's rows).
// A KV head with G query heads is nq pairs of G / nq heads, nq the smallest
// divisor of G with G / nq <= kMaxG: pair p of a sequence takes query heads
// p * G / nq .. + G / nq - 1 (rows stay contiguous) and reads KV head p / nq, so
// that KV head's cache is read nq times.
int head_groups(int G) {
  int nq = 1;
  while (G / nq > foscar::kMaxG || G % nq != 0) ++nq;
  return nq;
}
foscar_dims work_dims(const foscar_dims* d) {
  foscar_dims w = *d;
  w.num_kv_heads = d->num_kv_heads * head_groups(d->num_q_heads / d->num_kv_heads);
  return w;
}

int check_decode_shape(const foscar_dims* d, int layout, int group) {
  int rc = check_dims(d, true);
  if (rc) return rc;
  if (layout < 0 || layout > 15) return FOSCAR_EINVAL;  // K/V group sides and rotation bits
  if (!valid_group(group)) return FOSCAR_EUNSUPPORTED;
  // one grid row of work-groups per work pair; per-head byte offsets are 32-bit
  const int64_t pairs = (int64_t)d->batch * d->num_kv_heads * head_groups(d->num_q_heads / d->num_kv_heads);
  if (pairs > (1 << 22) || d->max_seq_len > (1 << 24)) return FOSCAR_EUNSUPPORTED;
  // a multiple of 32: a wave's last tile may then reach 32 tokens past Tcap, where every load reads
  // zero (each buffer resource ends at the KV head's last token) and the tokens are masked (t >= T)
  if (d->max_seq_len % 32 != 0) return FOSCAR_EUNSUPPORTED;
  if ((layout & 3) != 0 && d->max_seq_len % group != 0) return FOSCAR_EUNSUPPORTED;
  // a token-wise side groups g channels of a token
  if ((layout & 3) != (FOSCAR_K_CHANNEL | FOSCAR_V_CHANNEL) && d->head_dim % group != 0) return FOSCAR_EUNSUPPORTED;
  // rotated caches need head_dim 128 (Hadamard order of the kernels)
  if ((layout >> 2) != 0 && d->head_dim != foscar::kHeadDim) return FOSCAR_EUNSUPPORTED;
  return FOSCAR_OK;
}

// tokens one wave takes at a time
int unit_tokens(int layout, int group) { return (layout != 0 && group > foscar::kTile) ? group : foscar::kTile; }

int compute_units(int device) {
  std::lock_guard<std::mutex> lk(g_ws_mutex);
  auto it = g_cus.find(device);
  if (it != g_cus.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0) cus = 256;
  g_cus[device] = cus;
  return cus;
}

// Work-groups of the (bits, layout, group) kernel one CU of `device` holds at
// once (cached; 4 when the runtime cannot say, e.g. without a GPU).  `layout`
// may carry the rotation bits, which select the rotated variant.
int resident_per_cu(int device, int bits, int layout, int group, bool paged = false, int head_dim = foscar::kHeadDim) {
  const bool generic = head_dim != foscar::kHeadDim;  // the head-dim-generic kernels (their LDS depends on D)
  const long long key =
      (((((long long)device * 8 + bits) * 16 + layout) * 256 + group) * 2 + (paged ? 1 : 0)) * 512 + head_dim;
  {
    std::lock_guard<std::mutex> lk(g_ws_mutex);
    auto it = g_occ.find(key);
    if (it != g_occ.end()) return it->second;
  }
  int n = 0;
  const bool kch = (layout & FOSCAR_K_CHANNEL) != 0, vch = (layout & FOSCAR_V_CHANNEL) != 0;
  const hipError_t e = generic ? foscar::generic_occupancy(bits, kch, vch, group, head_dim, &n)
                               : foscar::decode_occupancy(bits, kch, vch, group, paged, (layout >> 2) != 0, &n);
  if (e != hipSuccess || n <= 0) return 4;
  std::lock_guard<std::mutex> lk(g_ws_mutex);
  g_occ[key] = n;
  return n;
}

// Split plan: one round of work-groups at the kernel's residency (more ranges
// only add per-range prologue, hand-off and merge work; measured), ranges of
// at most 4096 tokens so ragged batches balance, every range a multiple of the
// wave unit.
void plan(const foscar_dims* d, int layout, int group, int cus, int per_cu, int32_t* splits, int32_t* chunk,
          int extra_per_pair = 0, int max_chunk = 0) {
  const int unit = unit_tokens(layout, group);
  const int tcap = d->max_seq_len;
  const int units = (tcap + unit - 1) / unit;  // the last unit may reach past Tcap (by 32 tokens)
  if (units == 0) {
    *splits = 1;
    *chunk = unit;
    return;
  }
  const long long bh = (long long)d->batch * d->num_kv_heads;
  long long s = 1;
  const char* env = getenv("FOSCAR_SPLITS");
  if (env && atoi(env) > 0) {
    s = atoi(env);
  } else {
    // one round of resident work-groups, less the pairs' other work-groups (a fused window)
    const long long target = (long long)per_cu * cus - bh * extra_per_pair;
    if (bh > 0) s = std::max(1LL, (target + bh - 1) / bh);
    // but at least 8 tiles per wave: shorter ranges spend more on ramp-up, hand-off and merge
    // than they gain in parallel work (16 x 8192 tokens, INT2: 4 ranges 20.0 us, 8 ranges 22.1)
    s = std::min(s, std::max(1LL, (long long)tcap / (foscar::kTile * foscar::kWaves * 8)));
    // ranges of at most 4096 tokens: on ragged batches (lengths unknown to the host) shorter
    // ranges keep the last work-groups short; measured best for long and ragged caches
    const long long by_len = (tcap + 4095) / 4096;
    if (s < by_len) s = by_len;
  }
  if (s > foscar::kMaxSplits) s = foscar::kMaxSplits;
  // a paged cache: ranges of at most max_chunk tokens (the caller checks that this fits kMaxSplits)
  if (max_chunk > 0) s = std::max(s, ((long long)units + max_chunk / unit - 1) / (max_chunk / unit));
  if (s > units) s = units;
  if (s < 1) s = 1;
  const long long per = (units + s - 1) / s;
  *chunk = (int32_t)(per * unit);
  *splits = (int32_t)((units + per - 1) / per);
}

// A call needs one int32 counter per (sequence, KV head), padded to 256 B,
// and partials o_part fp32 [B*Hq*S*D] then lse_part fp32 [B*Hq*S].
size_t counter_bytes(const foscar_dims* d) {  // B*Hkv range counters, then the 2 work counters
  return (((size_t)d->batch * d->num_kv_heads + 2) * sizeof(int32_t) + 255) / 256 * 256;
}
size_t partial_bytes(const foscar_dims* d, int32_t splits) {  // range partials, then the window partials of each row
  const size_t rows = (size_t)d->batch * d->num_q_heads * (splits + foscar::kMaxWindowWgs);
  return rows * (d->head_dim + 1) * sizeof(float);
}

// Grow-only workspace of (current device, stream).  Growing frees the old
// buffer after synchronising the device, so no running call still uses it,
// and zeroes the new one.  *counters / *partials point into it.
int get_workspace(size_t cbytes, size_t pbytes, hipStream_t stream, int32_t** counters, float** partials) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lk(g_ws_mutex);
  Workspace& ws = g_ws[std::make_pair(dev, (void*)stream)];
  if (ws.counter_bytes < cbytes || ws.bytes - ws.counter_bytes < pbytes) {
    cbytes = std::max(cbytes, ws.counter_bytes);
    pbytes = std::max(pbytes, ws.bytes - ws.counter_bytes);
    const size_t bytes = cbytes + pbytes;
    if (ws.ptr) {
      e = hipDeviceSynchronize();
      if (e != hipSuccess) return hip_fail(e);
      (void)hipFree(ws.ptr);
      ws.ptr = nullptr;
      ws.bytes = 0;
      ws.counter_bytes = 0;
    }
    e = hipMalloc(&ws.ptr, bytes);
    if (e != hipSuccess) {
      ws.ptr = nullptr;
      return hip_fail(e);
    }
    // range counters must start at zero; every call leaves them at zero
    e = hipMemset(ws.ptr, 0, bytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      (void)hipFree(ws.ptr);
      ws.ptr = nullptr;
      return hip_fail(e);
    }
    ws.bytes = bytes;
    ws.counter_bytes = cbytes;
  }
  if (counters) *counters = (int32_t*)ws.ptr;
  if (partials) *partials = (float*)((char*)ws.ptr + ws.counter_bytes);
  return FOSCAR_OK;
}

// A workspace the caller provides instead of the grow-only one: counters (zero
// between calls, cbytes bytes at `base`) and partials (the rest, up to `bytes`).
struct FixedWorkspace {
  char* base = nullptr;
  size_t cbytes = 0;
  size_t bytes = 0;
};

// win_k == nullptr: no window.  Otherwise win_k, win_v bf16 [B][Hkv][win_cap][D] and win_lens [B].
// fixed != nullptr: run in that workspace (FOSCAR_ESCRATCH if the call needs more), allocate nothing.
int decode_common(int bits, const foscar_dims* d, const void* q, const void* pk, const void* pv, const void* ks,
                  const void* kz, const void* vs, const void* vz, const int32_t* seq_lens, int layout, int group,
                  void* out, float* lse, void* stream, bool windowed = false, const void* win_k = nullptr,
                  const void* win_v = nullptr, const int32_t* win_lens = nullptr, int32_t win_cap = 0,
                  const FixedWorkspace* fixed = nullptr, const int32_t* block_table = nullptr, int32_t block_size = 0,
                  int32_t num_blocks = 0) {
  const foscar::LaunchEvents ev = g_next_events;  // consumed by this call whether or not it launches
  g_next_events = foscar::LaunchEvents{};
  int rc = check_decode_shape(d, layout, group);
  if (rc) return rc;
  const bool generic = d->head_dim != foscar::kHeadDim;  // the head-dim-generic kernels: plain caches only
  if (generic && (windowed || block_table)) return FOSCAR_EUNSUPPORTED;
  const int rot = (layout >> 2) & 3;  // FOSCAR_K_ROTATED, FOSCAR_V_ROTATED
  const int variant = layout;         // the kernel variant (group sides and rotation)
  layout &= 3;                        // the group sides
  if (windowed) {
    if (win_cap < 0) return FOSCAR_EINVAL;
    if (win_cap > foscar::kMaxWindow || d->batch > 65535) return FOSCAR_EUNSUPPORTED;
  }
  if (d->batch == 0) return FOSCAR_OK;
  if (!q || !pk || !pv || !ks || !kz || !vs || !vz || !seq_lens || !out) return FOSCAR_EINVAL;
  if (windowed && win_cap > 0 && (!win_k || !win_v || !win_lens)) return FOSCAR_EINVAL;
  if (windowed && !win_lens) return FOSCAR_EINVAL;
  if (!aligned(pk, 16) || !aligned(pv, 16) || !aligned(ks, 16) || !aligned(kz, 16) || !aligned(vs, 16) ||
      !aligned(vz, 16) || !aligned(q, 4) || !aligned(seq_lens, 4) || !aligned(out, 4) || !aligned(lse, 4))
    return FOSCAR_EINVAL;
  if (windowed && (!aligned(win_k, 16) || !aligned(win_v, 16) || !aligned(win_lens, 4))) return FOSCAR_EINVAL;
  const bool paged = block_table != nullptr;
  const int hkv = d->num_kv_heads;

  const int kv_group = head_groups(d->num_q_heads / d->num_kv_heads);
  const foscar_dims wd = work_dims(d);
  d = &wd;  // from here on: work pairs (KV heads x kv_group)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  int32_t splits = 1, chunk = foscar::kTile;
  const int cus = compute_units(dev), per_cu = resident_per_cu(dev, bits, variant, group, paged, d->head_dim);
  // paged: the kernel's lanes hold one block each.  A range of at most 63 blocks' tokens touches at
  // most 64 blocks, aligned or not; when a block is the wave unit, every range starts on a block and
  // 64 blocks' tokens touch 64 (at P = 64, 4096-token ranges: one round of work-groups for a long
  // cache, where 4032-token ranges needed a second, nearly empty round)
  const int paged_blocks = block_size == unit_tokens(layout, group) ? 64 : 63;
  plan(d, layout, group, cus, per_cu, &splits, &chunk, 0, paged ? paged_blocks * block_size : 0);
  // the window is attended inside the decode launch by win_wgs more work-groups per pair: 1, 2, 4
  // or 8, with chunks of at most 4096 / 8 = 512 = kFusedWindowMax tokens.  A one-round grid has few
  // pairs: its window work-groups take chunks of at most 128 tokens where 8 allow it, beside the
  // ranges (planned for win_wgs slots fewer per pair).  A persistent grid has many pairs and runs
  // its window work-groups ahead of the round: there, fewer and longer chunks (up to 512 tokens)
  // keep their lanes busy (64 sequences x 8 KV heads, 1024-token window: 203 us per step against
  // 229 us with 128-token chunks)
  const bool one_round = (long long)splits * d->batch * d->num_kv_heads <= (long long)cus * per_cu ||
                         d->batch > foscar::kMapMaxB;
  const int win_target = one_round ? 128 : foscar::kFusedWindowMax;
  int win_wgs = 1;
  while (win_wgs < foscar::kMaxWindowWgs && win_wgs * win_target < win_cap) win_wgs *= 2;
  const int win_chunk = (win_cap + win_wgs - 1) / win_wgs;
  if (windowed && one_round) plan(d, layout, group, cus, per_cu, &splits, &chunk, win_wgs);
  int32_t* counters = nullptr;
  float* partials = nullptr;
  if (fixed) {
    if (counter_bytes(d) > fixed->cbytes || partial_bytes(d, splits) > fixed->bytes - fixed->cbytes)
      return FOSCAR_ESCRATCH;
    counters = (int32_t*)fixed->base;
    partials = (float*)(fixed->base + fixed->cbytes);
  } else {
    rc = get_workspace(counter_bytes(d), partial_bytes(d, splits), (hipStream_t)stream, &counters, &partials);
    if (rc) return rc;
  }

  const float sm = d->sm_scale > 0.f ? d->sm_scale : 1.0f / sqrtf((float)d->head_dim);
  if (generic) {
    foscar::GenericArgs ga;
    ga.q = (const uint16_t*)q;
    ga.pk = (const uint32_t*)pk;
    ga.pv = (const uint32_t*)pv;
    ga.ks = (const uint16_t*)ks;
    ga.kz = (const uint16_t*)kz;
    ga.vs = (const uint16_t*)vs;
    ga.vz = (const uint16_t*)vz;
    ga.seq_lens = seq_lens;
    ga.out = (uint16_t*)out;
    ga.lse = lse;
    ga.o_part = partials;
    ga.lse_part = partials + (size_t)d->batch * d->num_q_heads * splits * d->head_dim;
    ga.batch = d->batch;
    ga.hq = d->num_q_heads;
    ga.hkv = hkv;
    ga.pairs = d->num_kv_heads;  // work pairs per sequence
    ga.kv_group = kv_group;
    ga.g_heads = d->num_q_heads / d->num_kv_heads;
    ga.d = d->head_dim;
    ga.tcap = d->max_seq_len;
    ga.group = group;
    ga.splits = splits;
    ga.chunk = chunk;
    ga.sm_log2 = sm * 1.4426950408889634f;
    e = foscar::launch_decode_generic(bits, (layout & FOSCAR_K_CHANNEL) != 0, (layout & FOSCAR_V_CHANNEL) != 0, ga,
                                      (hipStream_t)stream, ev);
    return e == hipSuccess ? FOSCAR_OK : hip_fail(e);
  }
  foscar::SplitArgs sa;
  sa.q = (const uint16_t*)q;  // rotated keys: each work-group rotates its query rows (q H) itself
  sa.pk = (const uint32_t*)pk;
  sa.pv = (const uint32_t*)pv;
  sa.ks = (const uint16_t*)ks;
  sa.kz = (const uint16_t*)kz;
  sa.vs = (const uint16_t*)vs;
  sa.vz = (const uint16_t*)vz;
  sa.seq_lens = seq_lens;
  sa.out = (uint16_t*)out;
  sa.lse = lse;
  sa.counters = counters;
  sa.o_part = partials;
  sa.lse_part = sa.o_part + (size_t)d->batch * d->num_q_heads * splits * foscar::kHeadDim;
  sa.hq = d->num_q_heads;
  sa.hkv = d->num_kv_heads;
  sa.g_heads = d->num_q_heads / d->num_kv_heads;
  sa.kv_group = kv_group;
  sa.tcap = d->max_seq_len;
  sa.splits = splits;
  sa.chunk = chunk;
  sa.sm_log2 = sm * 1.4426950408889634f;
  // more work-groups than one round: a persistent round takes work items longest first
  sa.batch = d->batch;
  sa.grid_wgs = cus * per_cu;
  sa.persistent = ((long long)splits * d->batch * d->num_kv_heads > (long long)sa.grid_wgs &&
                   d->batch <= foscar::kMapMaxB) ? 1 : 0;
  sa.work_ctr = counters + (size_t)d->batch * d->num_kv_heads;
  sa.block_table = block_table;
  sa.block_size = block_size;
  sa.num_blocks = num_blocks;
  sa.win_o = nullptr;
  sa.win_lse = nullptr;
  sa.win_wgs = 0;
  sa.win_chunk = 0;
  sa.win_k = sa.win_v = nullptr;
  sa.win_lens = nullptr;
  sa.win_cap = 0;
  sa.win_sm = sm;
  sa.rot = rot;
  if (windowed) {  // beside the ranges (one round) or before the persistent round in the same grid
    const size_t rows = (size_t)d->batch * d->num_q_heads;
    sa.win_o = sa.lse_part + rows * splits;
    sa.win_lse = sa.win_o + rows * win_wgs * foscar::kHeadDim;
    sa.win_wgs = win_wgs;
    sa.win_chunk = win_chunk;
    sa.win_k = (const uint16_t*)win_k;
    sa.win_v = (const uint16_t*)win_v;
    sa.win_lens = win_lens;
    sa.win_cap = win_cap;
  }

  e = foscar::launch_decode(bits, (layout & FOSCAR_K_CHANNEL) != 0, (layout & FOSCAR_V_CHANNEL) != 0, group,
                            d->batch, d->num_kv_heads, sa, (hipStream_t)stream, ev);
  if (e != hipSuccess) return hip_fail(e);
  return FOSCAR_OK;
}

// ---------------------------------------------------------------------------
// Static scratch of the no-allocation entry point: the split workspace of
// foscar_decode_noalloc lives in this file-scope device array (one copy per
// GPU, held until the process ends).  [counters: kScratchCounterBytes][partials].
// Host code never passes the array's name to a kernel or a copy: it takes the
// device address from hipGetSymbolAddress once per device (scratch_on).
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(32) << 20;        // 32 MiB per GPU
constexpr size_t kScratchCounterBytes = size_t(64) << 10;  // 16384 counters (B * Hkv + 2)
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void zero_words(int32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

std::mutex g_scratch_mutex;
std::map<int, char*> g_scratch;  // device -> address of its copy of `scratch`

// Address of the current device's scratch; the first call on a device looks it
// up and clears its counter region with a fill kernel on `stream` (a kernel,
// not a memset, so that the call may be captured into a graph).
int scratch_on(hipStream_t stream, char** base) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lk(g_scratch_mutex);
  auto it = g_scratch.find(dev);
  if (it != g_scratch.end()) {
    *base = it->second;
    return FOSCAR_OK;
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
  const int n = (int)(kScratchCounterBytes / sizeof(int32_t));
  hipLaunchKernelGGL(zero_words, dim3((n + 255) / 256), dim3(256), 0, stream, (int32_t*)ptr, n);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  g_scratch[dev] = (char*)ptr;
  *base = (char*)ptr;
  return FOSCAR_OK;
}

int quantize_common(int bits, const foscar_dims* d, const void* k_src, const void* v_src, int32_t src_tokens,
                    const int32_t* start, const int32_t* count, int layout, int group, void* pk, void* pv, void* ks,
                    void* kz, void* vs, void* vz, void* stream) {
  int rc = check_dims(d, false);
  if (rc) return rc;
  if (d->head_dim != foscar::kHeadDim) return FOSCAR_EUNSUPPORTED;
  if (layout < 0 || layout > 15 || src_tokens < 0) return FOSCAR_EINVAL;
  const int rot = layout >> 2;  // FOSCAR_K_ROTATED, FOSCAR_V_ROTATED: rotate those rows first
  layout &= 3;
  if (!valid_group(group)) return FOSCAR_EUNSUPPORTED;
  if (d->max_seq_len % 32 != 0 || d->max_seq_len > (1 << 24)) return FOSCAR_EUNSUPPORTED;
  if (layout != 0 && d->max_seq_len % group != 0) return FOSCAR_EUNSUPPORTED;
  if (d->batch > 65535 || d->num_kv_heads > 65535) return FOSCAR_EUNSUPPORTED;  // grid z / y
  if (d->batch == 0 || src_tokens == 0) return FOSCAR_OK;
  if (!k_src || !v_src || !start || !count || !pk || !pv || !ks || !kz || !vs || !vz) return FOSCAR_EINVAL;
  if (!aligned(k_src, 16) || !aligned(v_src, 16) || !aligned(pk, 16) || !aligned(pv, 16) || !aligned(ks, 16) ||
      !aligned(kz, 16) || !aligned(vs, 16) || !aligned(vz, 16) || !aligned(start, 4) || !aligned(count, 4))
    return FOSCAR_EINVAL;
  const hipError_t e = foscar::launch_quantize(bits, (layout & FOSCAR_K_CHANNEL) != 0, (layout & FOSCAR_V_CHANNEL) != 0,
                                               group, rot, d->batch, d->num_kv_heads, d->max_seq_len, src_tokens, k_src,
                                               v_src, start, count, pk, pv, ks, kz, vs, vz, (hipStream_t)stream);
  return e == hipSuccess ? FOSCAR_OK : hip_fail(e);
}

int check_pack(int bits, int side, const foscar_dims* d) {
  if (bits != 2 && bits != 4) return FOSCAR_EINVAL;
  if (side != FOSCAR_SIDE_K && side != FOSCAR_SIDE_V) return FOSCAR_EINVAL;
  int rc = check_dims(d, false);
  if (rc) return rc;
  if (side == FOSCAR_SIDE_V && d->max_seq_len % (32 / bits) != 0) return FOSCAR_EUNSUPPORTED;
  return FOSCAR_OK;
}

}  // namespace

extern "C" {

int foscar_decode_int2(const foscar_dims* dims, const void* q, const void* packed_k, const void* packed_v,
                       const void* k_scale, const void* k_zero, const void* v_scale, const void* v_zero,
                       const int32_t* seq_lens, int layout, int group, void* out, float* lse, void* stream) {
  return decode_common(2, dims, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group,
                       out, lse, stream);
}

int foscar_decode_int4(const foscar_dims* dims, const void* q, const void* packed_k, const void* packed_v,
                       const void* k_scale, const void* k_zero, const void* v_scale, const void* v_zero,
                       const int32_t* seq_lens, int layout, int group, void* out, float* lse, void* stream) {
  return decode_common(4, dims, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group,
                       out, lse, stream);
}

int foscar_decode_window_int2(const foscar_dims* dims, const void* q, const void* packed_k, const void* packed_v,
                              const void* k_scale, const void* k_zero, const void* v_scale, const void* v_zero,
                              const int32_t* seq_lens, int layout, int group, const void* win_k, const void* win_v,
                              const int32_t* win_lens, int32_t win_cap, void* out, float* lse, void* stream) {
  return decode_common(2, dims, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group,
                       out, lse, stream, true, win_k, win_v, win_lens, win_cap);
}

int foscar_decode_window_int4(const foscar_dims* dims, const void* q, const void* packed_k, const void* packed_v,
                              const void* k_scale, const void* k_zero, const void* v_scale, const void* v_zero,
                              const int32_t* seq_lens, int layout, int group, const void* win_k, const void* win_v,
                              const int32_t* win_lens, int32_t win_cap, void* out, float* lse, void* stream) {
  return decode_common(4, dims, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group,
                       out, lse, stream, true, win_k, win_v, win_lens, win_cap);
}

int foscar_decode_noalloc(int bits, const foscar_dims* dims, const void* q, const void* packed_k,
                          const void* packed_v, const void* k_scale, const void* k_zero, const void* v_scale,
                          const void* v_zero, const int32_t* seq_lens, int layout, int group, void* out, float* lse,
                          void* stream) {
  if (bits != 2 && bits != 4) return FOSCAR_EINVAL;
  int rc = check_decode_shape(dims, layout, group);
  if (rc) return rc;
  if (dims->batch == 0) return FOSCAR_OK;
  // sizes the static scratch cannot hold fail before any HIP call: the counters, and the
  // partials of the smallest plan (one range per pair)
  const foscar_dims wd = work_dims(dims);
  if (counter_bytes(&wd) > kScratchCounterBytes || partial_bytes(&wd, 1) > kScratchBytes - kScratchCounterBytes)
    return FOSCAR_ESCRATCH;
  if (!q || !packed_k || !packed_v || !k_scale || !k_zero || !v_scale || !v_zero || !seq_lens || !out)
    return FOSCAR_EINVAL;
  char* base = nullptr;
  rc = scratch_on((hipStream_t)stream, &base);
  if (rc) return rc;
  FixedWorkspace ws;
  ws.base = base;
  ws.cbytes = kScratchCounterBytes;
  ws.bytes = kScratchBytes;
  return decode_common(bits, dims, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group,
                       out, lse, stream, false, nullptr, nullptr, nullptr, 0, &ws);
}

namespace {
int decode_paged(int bits, const foscar_dims* dims, const void* q, const void* k_pool, const void* v_pool,
                 const void* k_scale, const void* k_zero, const void* v_scale, const void* v_zero,
                 const int32_t* block_table, int32_t block_size, int32_t num_blocks, const int32_t* seq_lens,
                 int layout, int group, void* out, float* lse, void* stream) {
  int rc = check_decode_shape(dims, layout, group);
  if (rc) return rc;
  if (dims->head_dim != foscar::kHeadDim) return FOSCAR_EUNSUPPORTED;
  if (!block_table || !aligned(block_table, 4) || num_blocks < 1 || block_size < 1) return FOSCAR_EINVAL;
  // blocks of whole tiles (and whole groups of a channel-wise side); the logical capacity
  // max_seq_len is a whole number of blocks, in at most kMaxSplits ranges of 63 blocks' tokens
  if (block_size % foscar::kTile != 0 || block_size > 65536) return FOSCAR_EUNSUPPORTED;
  if ((layout & 3) != 0 && block_size % group != 0) return FOSCAR_EUNSUPPORTED;
  if (dims->max_seq_len % block_size != 0) return FOSCAR_EUNSUPPORTED;
  if ((int64_t)dims->max_seq_len > (int64_t)foscar::kMaxSplits * 63 * block_size) return FOSCAR_EUNSUPPORTED;
  return decode_common(bits, dims, q, k_pool, v_pool, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group, out,
                       lse, stream, false, nullptr, nullptr, nullptr, 0, nullptr, block_table, block_size, num_blocks);
}
}  // namespace

int foscar_decode_paged_int2(const foscar_dims* dims, const void* q, const void* k_pool, const void* v_pool,
                             const void* k_scale, const void* k_zero, const void* v_scale, const void* v_zero,
                             const int32_t* block_table, int32_t block_size, int32_t num_blocks,
                             const int32_t* seq_lens, int layout, int group, void* out, float* lse, void* stream) {
  return decode_paged(2, dims, q, k_pool, v_pool, k_scale, k_zero, v_scale, v_zero, block_table, block_size,
                      num_blocks, seq_lens, layout, group, out, lse, stream);
}

int foscar_decode_paged_int4(const foscar_dims* dims, const void* q, const void* k_pool, const void* v_pool,
                             const void* k_scale, const void* k_zero, const void* v_scale, const void* v_zero,
                             const int32_t* block_table, int32_t block_size, int32_t num_blocks,
                             const int32_t* seq_lens, int layout, int group, void* out, float* lse, void* stream) {
  return decode_paged(4, dims, q, k_pool, v_pool, k_scale, k_zero, v_scale, v_zero, block_table, block_size,
                      num_blocks, seq_lens, layout, group, out, lse, stream);
}

int foscar_quantize_int2(const foscar_dims* dims, const void* k_src, const void* v_src, int32_t src_tokens,
                         const int32_t* start, const int32_t* count, int layout, int group, void* packed_k,
                         void* packed_v, void* k_scale, void* k_zero, void* v_scale, void* v_zero, void* stream) {
  return quantize_common(2, dims, k_src, v_src, src_tokens, start, count, layout, group, packed_k, packed_v, k_scale,
                         k_zero, v_scale, v_zero, stream);
}

int foscar_quantize_int4(const foscar_dims* dims, const void* k_src, const void* v_src, int32_t src_tokens,
                         const int32_t* start, const int32_t* count, int layout, int group, void* packed_k,
                         void* packed_v, void* k_scale, void* k_zero, void* v_scale, void* v_zero, void* stream) {
  return quantize_common(4, dims, k_src, v_src, src_tokens, start, count, layout, group, packed_k, packed_v, k_scale,
                         k_zero, v_scale, v_zero, stream);
}

int foscar_pack(int bits, int side, const foscar_dims* dims, const uint8_t* codes, void* packed, void* stream) {
  int rc = check_pack(bits, side, dims);
  if (rc) return rc;
  if ((size_t)dims->batch * dims->num_kv_heads * dims->max_seq_len == 0) return FOSCAR_OK;
  if (!codes || !packed) return FOSCAR_EINVAL;
  hipError_t e = foscar::launch_pack(bits, side, dims->batch, dims->num_kv_heads, dims->max_seq_len, dims->head_dim,
                                     codes, (uint32_t*)packed, (hipStream_t)stream);
  return e == hipSuccess ? FOSCAR_OK : hip_fail(e);
}

int foscar_unpack(int bits, int side, const foscar_dims* dims, const void* packed, uint8_t* codes, void* stream) {
  int rc = check_pack(bits, side, dims);
  if (rc) return rc;
  if ((size_t)dims->batch * dims->num_kv_heads * dims->max_seq_len == 0) return FOSCAR_OK;
  if (!codes || !packed) return FOSCAR_EINVAL;
  hipError_t e = foscar::launch_unpack(bits, side, dims->batch, dims->num_kv_heads, dims->max_seq_len, dims->head_dim,
                                       (const uint32_t*)packed, codes, (hipStream_t)stream);
  return e == hipSuccess ? FOSCAR_OK : hip_fail(e);
}

size_t foscar_packed_bytes(int bits, int side, const foscar_dims* dims) {
  if (check_pack(bits, side, dims)) return 0;
  return (size_t)dims->batch * dims->num_kv_heads * dims->max_seq_len * dims->head_dim * bits / 8;
}

size_t foscar_scale_count(int side, int side_layout, int group, const foscar_dims* dims) {
  if (check_dims(dims, false) || !valid_group(group)) return 0;
  if (side != FOSCAR_SIDE_K && side != FOSCAR_SIDE_V) return 0;
  const int channel_bit = side == FOSCAR_SIDE_K ? FOSCAR_K_CHANNEL : FOSCAR_V_CHANNEL;
  if (side_layout != 0 && side_layout != channel_bit) return 0;
  const size_t bh = (size_t)dims->batch * dims->num_kv_heads;
  if (side_layout == 0) return bh * dims->max_seq_len * (dims->head_dim / group);
  if (dims->max_seq_len % group) return 0;
  return bh * (dims->max_seq_len / group) * dims->head_dim;
}

int foscar_split_plan(const foscar_dims* dims, int bits, int layout, int group, int32_t* splits, int32_t* chunk) {
  int rc = check_decode_shape(dims, layout, group);
  if (rc) return rc;
  if (bits != 2 && bits != 4) return FOSCAR_EINVAL;
  if (!splits || !chunk) return FOSCAR_EINVAL;
  int dev = 0, cus = 256, per_cu = 4;
  if (hipGetDevice(&dev) == hipSuccess) {
    cus = compute_units(dev);
    per_cu = resident_per_cu(dev, bits, layout, group, false, dims->head_dim);
  }
  const foscar_dims wd = work_dims(dims);
  plan(&wd, layout & 3, group, cus, per_cu, splits, chunk);
  return FOSCAR_OK;
}

int foscar_record_next_launch(void* start_event, void* stop_event) {
  g_next_events.start = (hipEvent_t)start_event;
  g_next_events.stop = (hipEvent_t)stop_event;
  return FOSCAR_OK;
}

int foscar_occupancy(int bits, int layout, int group, int32_t* wgs_per_cu) {
  if (!wgs_per_cu) return FOSCAR_EINVAL;
  if (layout < 0 || layout > 15) return FOSCAR_EINVAL;
  if ((bits != 2 && bits != 4) || !valid_group(group)) return FOSCAR_EUNSUPPORTED;
  int n = 0;
  const hipError_t e = foscar::decode_occupancy(bits, (layout & FOSCAR_K_CHANNEL) != 0, (layout & FOSCAR_V_CHANNEL) != 0,
                                                group, false, (layout >> 2) != 0, &n);
  if (e != hipSuccess) return hip_fail(e);
  *wgs_per_cu = n;
  return FOSCAR_OK;
}

int foscar_workspace_reserve(const foscar_dims* dims, int bits, int layout, int group, void* stream) {
  int rc = check_decode_shape(dims, layout, group);
  if (rc) return rc;
  if (bits != 2 && bits != 4) return FOSCAR_EINVAL;
  if (dims->batch == 0) return FOSCAR_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  int32_t splits = 1, chunk = 0;
  const foscar_dims wd = work_dims(dims);
  plan(&wd, layout & 3, group, compute_units(dev),
       resident_per_cu(dev, bits, layout, group, false, dims->head_dim), &splits, &chunk);
  return get_workspace(counter_bytes(&wd), partial_bytes(&wd, splits), (hipStream_t)stream, nullptr, nullptr);
}

void foscar_release(void) {
  std::lock_guard<std::mutex> lk(g_ws_mutex);
  if (g_ws.empty()) return;
  int cur = 0;
  bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (auto& kv : g_ws) {
    if (!kv.second.ptr) continue;
    if (hipSetDevice(kv.first.first) == hipSuccess) {
      (void)hipDeviceSynchronize();
      (void)hipFree(kv.second.ptr);
    }
  }
  g_ws.clear();
  if (have_cur) (void)hipSetDevice(cur);
}

const char* foscar_strerror(int code) {
  switch (code) {
    case FOSCAR_OK: return "ok";
    case FOSCAR_EINVAL: return "invalid argument";
    case FOSCAR_EUNSUPPORTED: return "unsupported shape or parameter";
    case FOSCAR_EHIP: return "HIP runtime error";
    case FOSCAR_ENOMEM: return "out of device memory";
    case FOSCAR_ESCRATCH: return "call needs more than the static scratch of the no-allocation entry point";
  }
  return "unknown error";
}

int foscar_version(void) { return FOSCAR_VERSION; }

int foscar_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
