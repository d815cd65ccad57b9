/*
 * foscar.h -- decode attention over a 2-bit or 4-bit quantised KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the one of "FOSCAR: Accelerating Decode Attention over 2- and
 * 4-Bit KV Caches through Affine Folding" (arXiv 2611.09722; abstract) and of
 * its explainer "FOSCAR speeds up 2-bit KV decode -- Affine folding of KV
 * dequantization" (learnaivisually):
 *   - the cache holds codes q with one scale s and one offset z per group,
 *     value = s*q + z (explainer, encoding paragraph);
 *   - groups run token-wise (g channels of one token) or channel-wise (g
 *     tokens of one channel) (explainer, fold-placement table);
 *   - no value is dequantised one by one: token-wise K and channel-wise V scale
 *     each group's partial sum once (acc-fold), channel-wise K and token-wise V
 *     pre-scale the other operand (operand-fold); each offset becomes one
 *     correction z * (sum of the other operand) (explainer, fold rule and
 *     table); key-side corrections land before the softmax, value-side ones
 *     before the final division (explainer, fold rule).
 * The result equals softmax attention over the dequantised cache, up to
 * floating-point rounding (abstract: exact in exact arithmetic).
 *
 * One decode step = one new query token per sequence, grouped-query
 * attention: query head i reads KV head i / (Hq / Hkv).
 *
 * Conventions for every entry point:
 *   - all tensor pointers are DEVICE memory owned by the caller; inputs are
 *     only read; the library never frees or keeps them;
 *   - packed codes, scales, offsets, bf16 key/value sources and windows must
 *     be 16-byte aligned, every other tensor 4-byte aligned (FOSCAR_EINVAL
 *     otherwise); fresh allocations are;
 *   - `stream` is a hipStream_t (NULL = the null stream of the current
 *     device); calls are asynchronous on it: no host synchronisation and no
 *     host read of device data; buffers must stay alive until the stream has
 *     passed the call;
 *   - arguments are validated on the host BEFORE any HIP call; an invalid
 *     call returns an error code and launches nothing;
 *   - return value: FOSCAR_OK (0) or a negative FOSCAR_E* code; no exception
 *     or abort crosses this interface.
 */
#ifndef FOSCAR_H
#define FOSCAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FOSCAR_VERSION 100 /* 1.0.0 */

/* Return codes. */
#define FOSCAR_OK 0
#define FOSCAR_EINVAL (-1)       /* null or misaligned pointer, negative size, bad layout/side/bits value,
                                    Hq % Hkv != 0 */
#define FOSCAR_EUNSUPPORTED (-2) /* head_dim not 128 where 128 is required (window, paged, rotated,
                                    quantise) or not a multiple of 32 up to 256, a token-wise
                                    group that does not divide head_dim,
                                    group not in {32,64,128}, Hq/Hkv > 16,
                                    max_seq_len not a multiple of 32 (and of group for a
                                    channel-wise side), max_seq_len > 2^24,
                                    batch * num_kv_heads > 2^22 */
#define FOSCAR_EHIP (-3)         /* a HIP call failed; foscar_last_hip_error() has its code */
#define FOSCAR_ENOMEM (-4)       /* workspace allocation failed */
#define FOSCAR_ESCRATCH (-5)     /* foscar_decode_noalloc: the call needs more split workspace than the
                                    library's static scratch holds */

/* Layout bits (OR one K value with one V value).
 * Token-wise group: g consecutive channels of one token share (s, z).
 * Channel-wise group: g consecutive tokens (from token 0) of one channel share (s, z). */
#define FOSCAR_K_TOKEN 0
#define FOSCAR_K_CHANNEL 1
#define FOSCAR_V_TOKEN 0
#define FOSCAR_V_CHANNEL 2
/* Rotated cache (OR with the bits above).  The
 * accuracy recipe the explainer's accuracy paragraph names ("OSCAR's
 * rotations"; its related explainers: KVarN, a Hadamard-rotated 2-bit KV
 * cache): the cache holds the quantised rows of K H and/or V H, H the
 * orthonormal Sylvester-Hadamard matrix of order 128 (entry (i, j) =
 * (-1)^popcount(i & j) / sqrt(128); symmetric, H H = I).
 *   FOSCAR_K_ROTATED: the keys are rotated; each work-group rotates the query
 *     rows it attends with (q H, rounded once to bf16 from an fp64 transform
 *     whose sums are exact) before they meet the keys, so the scores are those
 *     of q against K.
 *   FOSCAR_V_ROTATED: the values are rotated; the cache's weighted value sum is
 *     taken back by H (fp32) before the final division, so `out` is in the
 *     model's basis.
 * A full-precision window (foscar_decode_window_*) holds unrotated rows and
 * meets the query itself.  The rotated query must lie in the fp16 range. */
/* For foscar_quantize_int2/int4 the same bits rotate the new key / value rows
 * (x H: fp64 butterflies, exact for bf16 values, one rounding to fp32) before
 * they are quantised, so that the cache holds the rows the decode expects. */
#define FOSCAR_K_ROTATED 4
#define FOSCAR_V_ROTATED 8

/* Sides for pack / unpack / sizing. */
#define FOSCAR_SIDE_K 0
#define FOSCAR_SIDE_V 1

typedef struct foscar_dims {
  int32_t batch;        /* B >= 0 sequences (B = 0: nothing to do) */
  int32_t num_q_heads;  /* Hq >= 1 */
  int32_t num_kv_heads; /* Hkv >= 1, Hq % Hkv == 0, G = Hq / Hkv <= 16 (see foscar_decode_int2) */
  int32_t head_dim;     /* D: 128 for every entry point; foscar_decode_int2/int4, foscar_decode_noalloc,
                           pack/unpack and the sizes also take a multiple of 32 up to 256 */
  int32_t max_seq_len;  /* Tcap: tokens allocated per sequence; multiple of 32, and of
                           `group` when a side is channel-wise */
  float sm_scale;       /* softmax scale applied to q.k; <= 0 selects 1/sqrt(head_dim) */
} foscar_dims;

/*
 * Decode step, 2-bit (foscar_decode_int2) or 4-bit (foscar_decode_int4) codes.
 *
 * q         bf16  [B][Hq][D]; query head i attends KV head i / G, G = Hq / Hkv <= 16.
 *           A KV head is read once per group of at most 4 of its query heads
 *           (G = 8: twice, G = 16: four times; G prime above 4: G times).
 * packed_k  u32   [B][Hkv][Tcap][D*bits/32]   keys packed along channels
 * packed_v  u32   [B][Hkv][Tcap*bits/32][D]   values packed along tokens
 *           E = 32/bits codes per word; word holds E consecutive elements of the
 *           packed axis; element e of a word sits at bits
 *           [bits*(e/2) + 16*(e%2), +bits): even elements in the low half-word,
 *           odd elements in the high half-word (little-endian, lowest bits first).
 *           Codes are unsigned, 0 .. 2^bits - 1.
 * k_scale, k_zero  fp16, token-wise [B][Hkv][Tcap][D/g], channel-wise [B][Hkv][Tcap/g][D]
 * v_scale, v_zero  fp16, same two shapes for the value side
 * seq_lens  int32 [B]; T_b is clamped on the device to [0, Tcap].  Tokens at or
 *           past T_b (codes, scales, offsets) may hold anything, NaN included,
 *           and do not affect the result.  A channel-wise group that reaches
 *           past T_b covers only its tokens below T_b.
 * layout    FOSCAR_K_* | FOSCAR_V_* (| FOSCAR_K_ROTATED | FOSCAR_V_ROTATED)
 * group     g in {32, 64, 128} (channels for a token-wise side, tokens for a
 *           channel-wise side; the same g for both sides)
 * out       bf16  [B][Hq][D]  softmax(sm_scale * q K^T) V over the dequantised
 *           cache, rounded to nearest even; 0 for a row with T_b = 0
 * lse       fp32  [B][Hq]     ln sum_t exp(sm_scale * q.k_t); -inf when T_b = 0
 *           (may be NULL)
 * stream    hipStream_t
 *
 * Head dims other than 128 (a multiple of 32 up to 256; plain layouts, no
 * rotation bits; a token-wise side's g must divide D) run on a second pair of
 * kernels with the same folds (fold-placement table of the FOSCAR explainer)
 * on the vector ALUs: token-wise keys as fp16 dot products of the query
 * (exact for bf16 values in the fp16 range) and the codes, channel-wise keys
 * as fp32 products of q * s and the codes, value sums as fp16 dot products of
 * the weights (p, or p * s for a token-wise value side) and the codes, all
 * accumulated in fp32; one launch writes each range's partial, a second merges
 * them.  Their results meet the same error bound; their speed is not that of
 * the D = 128 kernels.
 *
 * Precision (D = 128): token-wise keys: q K^T on the block-scaled matrix cores, the
 * query as two e4m3 terms (exact for bf16 values) times the key codes (exact),
 * products summed in the matrix core to about 14 significant bits of each
 * 16-token block's largest product, fp32 beyond; channel-wise keys: fp16
 * products (query times scale as an exact fp16 pair), fp32 accumulation.  P V:
 * fp16 weights (softmax weights, times the value scale for a token-wise value
 * side) times the value codes, fp32 accumulation.  Query values must lie in the
 * fp16 range; value scales of a token-wise value side must satisfy |s| < 256.  The first call on a (device, stream) pair may allocate the
 * split workspace (see foscar_workspace_reserve); later calls of the same or
 * smaller size do not allocate.  Calls on different streams do not share
 * workspace.
 */
int foscar_decode_int2(const foscar_dims* dims, const void* q, const void* packed_k, const void* packed_v,
                       const void* k_scale, const void* k_zero, const void* v_scale, const void* v_zero,
                       const int32_t* seq_lens, int layout, int group, void* out, float* lse, void* stream);
int foscar_decode_int4(const foscar_dims* dims, const void* q, const void* packed_k, const void* packed_v,
                       const void* k_scale, const void* k_zero, const void* v_scale, const void* v_zero,
                       const int32_t* seq_lens, int layout, int group, void* out, float* lse, void* stream);

/*
 * Decode step that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Arguments and results as foscar_decode_int2 (bits = 2)
 * or foscar_decode_int4 (bits = 4), same kernels and split plan; the caller
 * passes every input and output.
 *
 * The split workspace (range counters and partial results) is a static device
 * array of 32 MiB inside the library, one copy per GPU, held until the process
 * ends: 64 KiB of counters (batch * num_kv_heads + 2 of them) and the rest for
 * partials, batch * num_q_heads * (splits + 8) * (head_dim + 1) floats.  A call that needs
 * more returns FOSCAR_ESCRATCH: before any HIP call when even one range per
 * (sequence, KV head) does not fit, otherwise after planning, still before
 * any launch.  No call here allocates or frees device memory; the first call
 * on a device looks up the array's address and clears its counters with a
 * small kernel on `stream`.  Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (different streams, or different host
 * threads) race and must be serialised by the caller; calls on one stream
 * are ordered and never race.  Each call leaves the counters at zero.
 */
int foscar_decode_noalloc(int bits, const foscar_dims* dims, const void* q, const void* packed_k,
                          const void* packed_v, const void* k_scale, const void* k_zero, const void* v_scale,
                          const void* v_zero, const int32_t* seq_lens, int layout, int group, void* out, float* lse,
                          void* stream);

/*
 * Decode step over the quantised cache plus a full-precision window of recent
 * tokens (2-bit: foscar_decode_window_int2, 4-bit: foscar_decode_window_int4).
 *
 * The FOSCAR explainer's accuracy paragraph names full-precision windows of
 * recent tokens as part of the accuracy recipe a 2-bit cache needs.  The
 * window's tokens are further keys and values of the same softmax: out and lse
 * are those of attention over the T_b cache tokens and the window's tokens
 * together.  The window is attended in fp32 from bf16 by 1-8 extra
 * work-groups per (sequence, KV head) of the decode launch itself, and merged
 * with the cache's ranges by log-sum-exp inside the same kernel: one launch per
 * call.
 *
 * Arguments as foscar_decode_int2/int4, plus:
 * win_k, win_v  bf16 [B][Hkv][win_cap][D]: window keys and values
 * win_lens      int32 [B] (device): window tokens of each sequence, clamped to
 *               [0, win_cap]; rows past them may hold anything
 * win_cap       0 .. 4096 tokens (win_k / win_v may be NULL when 0)
 * A sequence with no cache token and no window token gives out = 0,
 * lse = -inf.  The window uses slots of the split workspace (see
 * foscar_workspace_reserve, which reserves them).
 */
int foscar_decode_window_int2(const foscar_dims* dims, const void* q, const void* packed_k, const void* packed_v,
                              const void* k_scale, const void* k_zero, const void* v_scale, const void* v_zero,
                              const int32_t* seq_lens, int layout, int group, const void* win_k, const void* win_v,
                              const int32_t* win_lens, int32_t win_cap, void* out, float* lse, void* stream);
int foscar_decode_window_int4(const foscar_dims* dims, const void* q, const void* packed_k, const void* packed_v,
                              const void* k_scale, const void* k_zero, const void* v_scale, const void* v_zero,
                              const int32_t* seq_lens, int layout, int group, const void* win_k, const void* win_v,
                              const int32_t* win_lens, int32_t win_cap, void* out, float* lse, void* stream);

/*
 * Decode step over a paged cache (2-bit: foscar_decode_paged_int2, 4-bit:
 * foscar_decode_paged_int4): the cache of every sequence is a list of blocks
 * of block_size tokens taken from shared pools through a block table, the
 * layout of serving systems whose prefix cache shares blocks between requests
 * (the FOSCAR explainer's integration paragraph names SGLang, which keeps its
 * KV cache this way).  Attention is the same as foscar_decode_int2/int4 over
 * the sequence's tokens in logical order.
 *
 * Arguments as foscar_decode_int2/int4, except:
 * k_pool, v_pool, k_scale, k_zero, v_scale, v_zero
 *              pools of num_blocks blocks: each array's layout of
 *              foscar_decode_int2 with B = num_blocks and Tcap = block_size,
 *              e.g. k_pool u32 [num_blocks][Hkv][block_size][D*bits/32],
 *              v_pool u32 [num_blocks][Hkv][block_size*bits/32][D], token-wise
 *              scales [num_blocks][Hkv][block_size][D/g], channel-wise
 *              [num_blocks][Hkv][block_size/g][D] (a channel-wise group never
 *              crosses a block)
 * block_table  int32 [B][max_seq_len / block_size] (device): logical block j of
 *              sequence b (tokens j*block_size ..) is pool block
 *              block_table[b][j]; entries of blocks at or past T_b are not read
 *              as block ids (they may hold anything); an entry outside
 *              [0, num_blocks) of a block below T_b reads that block as zeros
 * block_size   a multiple of 64 (and of g for a channel-wise side), <= 65536;
 *              max_seq_len is a whole number of blocks, at most
 *              512 * 63 * block_size tokens
 * num_blocks   >= 1
 * Errors: FOSCAR_EINVAL for a null or misaligned block_table, num_blocks < 1;
 * FOSCAR_EUNSUPPORTED for a block_size or max_seq_len outside the rules above.
 */
int foscar_decode_paged_int2(const foscar_dims* dims, const void* q, const void* k_pool, const void* v_pool,
                             const void* k_scale, const void* k_zero, const void* v_scale, const void* v_zero,
                             const int32_t* block_table, int32_t block_size, int32_t num_blocks,
                             const int32_t* seq_lens, int layout, int group, void* out, float* lse, void* stream);
int foscar_decode_paged_int4(const foscar_dims* dims, const void* q, const void* k_pool, const void* v_pool,
                             const void* k_scale, const void* k_zero, const void* v_scale, const void* v_zero,
                             const int32_t* block_table, int32_t block_size, int32_t num_blocks,
                             const int32_t* seq_lens, int layout, int group, void* out, float* lse, void* stream);

/*
 * Quantise new keys and values into the cache (2-bit: foscar_quantize_int2,
 * 4-bit: foscar_quantize_int4), in the layouts the decode entry points read.
 *
 * Encoding value = s*q + z, one (s, z) per group (explainer, encoding
 * paragraph); groups token-wise or channel-wise as in `layout` (explainer,
 * fold-placement table).  The pages give no quantiser; this one is min-max
 * asymmetric with every decision in fp32:
 *   s = fp16_rne(fp32(max - min) / (2^bits - 1)),  z = fp16_rne(min),
 *   q = clamp(rint_half_even(fp32(x - z) / s), 0, 2^bits - 1), q = 0 if s = 0.
 *
 * k_src, v_src  bf16 [B][Hkv][src_tokens][D]: row r of sequence b is token
 *               start[b] + r; finite values with |x| < 65504
 * start, count  int32 [B] (device): sequence b receives tokens
 *               [start[b], start[b] + n_b), n_b = count[b] clamped to
 *               [0, min(src_tokens, Tcap - start[b])]; start[b] outside
 *               [0, Tcap] leaves the sequence untouched
 * layout, group as for decode (with FOSCAR_K_ROTATED / FOSCAR_V_ROTATED, the
 *               rows of that side are rotated first).  A token-wise side quantises each token's
 *               groups of g channels.  A channel-wise side needs start[b] to
 *               be a multiple of g (otherwise sequence b is left untouched);
 *               each group g*tau .. g*tau + g - 1 the range reaches is
 *               quantised over the tokens of the range it holds (a partly
 *               filled last group is quantised over its tokens so far and is
 *               re-quantised whole by a later call that starts at g*tau).
 * packed_k, packed_v, k_scale, k_zero, v_scale, v_zero
 *               the cache, in the layouts of the decode entry points; only
 *               the written tokens' codes and their groups' (s, z) change:
 *               codes of other tokens in a shared value word are kept.
 * Only batch, num_kv_heads, head_dim and max_seq_len of dims are used
 * (head_dim 128; max_seq_len a multiple of 32, and of g for a channel-wise
 * side; batch and num_kv_heads at most 65535).
 * Asynchronous on `stream`; the caller keeps the buffers alive.  Calls that
 * write the same sequences must be ordered on one stream.
 */
int foscar_quantize_int2(const foscar_dims* dims, const void* k_src, const void* v_src, int32_t src_tokens,
                         const int32_t* start, const int32_t* count, int layout, int group, void* packed_k,
                         void* packed_v, void* k_scale, void* k_zero, void* v_scale, void* v_zero, void* stream);
int foscar_quantize_int4(const foscar_dims* dims, const void* k_src, const void* v_src, int32_t src_tokens,
                         const int32_t* start, const int32_t* count, int layout, int group, void* packed_k,
                         void* packed_v, void* k_scale, void* k_zero, void* v_scale, void* v_zero, void* stream);

/*
 * Pack logical codes into the layout above (bit-exact with any packer written
 * from the same specification), or unpack it.
 * codes   u8 [B][Hkv][Tcap][D], values 0 .. 2^bits - 1 (higher bits are dropped)
 * packed  u32, FOSCAR_SIDE_K: [B][Hkv][Tcap][D*bits/32]; FOSCAR_SIDE_V: [B][Hkv][Tcap*bits/32][D]
 * bits    2 or 4;  side  FOSCAR_SIDE_K or FOSCAR_SIDE_V
 * Only batch, num_kv_heads, head_dim and max_seq_len of dims are used
 * (head_dim 128 or a multiple of 32 up to 256, max_seq_len a multiple of 32/bits for FOSCAR_SIDE_V).
 */
int foscar_pack(int bits, int side, const foscar_dims* dims, const uint8_t* codes, void* packed, void* stream);
int foscar_unpack(int bits, int side, const foscar_dims* dims, const void* packed, uint8_t* codes, void* stream);

/* Bytes of one packed side (pure host arithmetic; 0 on invalid arguments). */
size_t foscar_packed_bytes(int bits, int side, const foscar_dims* dims);

/* Number of fp16 scales (equally offsets) of one side:
 * side_layout is FOSCAR_K_TOKEN/FOSCAR_K_CHANNEL for side K (pass side = FOSCAR_SIDE_K)
 * or FOSCAR_V_TOKEN/FOSCAR_V_CHANNEL for side V; 0 on invalid arguments. */
size_t foscar_scale_count(int side, int side_layout, int group, const foscar_dims* dims);

/*
 * Allocate (grow-only) the split workspace that decode calls with these dims,
 * bits (2 or 4), layout and group use on `stream` of the current device, so
 * that no later call of that size allocates.  Synchronous.  FOSCAR_ENOMEM on
 * failure.
 */
int foscar_workspace_reserve(const foscar_dims* dims, int bits, int layout, int group, void* stream);

/* Free every workspace of the library (all devices and streams).  The caller
 * must make sure no decode call is still running.  Synchronous. */
void foscar_release(void);

/* Split plan the decode entry points use for these arguments (bits 2 or 4),
 * without a window: *splits = number of key/value ranges per (sequence, KV
 * head), *chunk = tokens per range.  The plan fills the device once at the
 * kernel's residency (foscar_occupancy), keeps at least 8 tiles of 64 tokens
 * per wave and makes ranges of at most 4096 tokens.  A windowed call whose
 * grid runs in one round plans its ranges for the slots its window
 * work-groups leave.
 * FOSCAR_SPLITS=<n> in the environment forces n ranges (tuning and tests);
 * the count is capped at 512 ranges and at one range per 64-token unit. */
int foscar_split_plan(const foscar_dims* dims, int bits, int layout, int group, int32_t* splits, int32_t* chunk);

/* Timing: the next foscar_decode_int2/int4 call on this host thread records
 * start_event / stop_event (hipEvent_t created by the caller; either may be
 * NULL) as part of its kernel dispatch, so their elapsed time is the decode
 * kernel's own duration, without the queue's gaps around it.  The request is
 * consumed by that call whether or not it launches (an empty batch or an
 * argument error launches nothing).  Always FOSCAR_OK. */
int foscar_record_next_launch(void* start_event, void* stop_event);

/* Work-groups of the decode kernel for (bits, layout, group) that one compute
 * unit of the current device holds at once (registers and LDS permitting).
 * Reporting only; FOSCAR_EUNSUPPORTED for bits/group outside the supported
 * set, FOSCAR_EHIP if the runtime query fails. */
int foscar_occupancy(int bits, int layout, int group, int32_t* wgs_per_cu);

const char* foscar_strerror(int code);
int foscar_version(void);
/* hipError_t of the last failed HIP call on this host thread (0 if none). */
int foscar_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FOSCAR_H */
