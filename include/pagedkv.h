/*
 * pagedkv.h -- C ABI of the MI355X (gfx950) paged KV cache library.
 *
 * Three operations make up the hot path of a paged KV cache in a dense GQA
 * decoder such as Qwen3-0.6B:
 *   pa_reshape_and_cache      token-major K/V -> paged cache, through a slot
 *                             mapping (optional SWA remap, optional fp8 scale)
 *   pa_concat_and_cast_mla_k  per-head k_nope ++ shared k_rope -> K, with a cast
 *   pa_concat_and_cache_mla_k the same K assembled straight into the paged cache
 *   pa_decode_attention       one query token per sequence against its paged
 *                             K/V, read back through a block table (GQA)
 *   pa_decode_step            the new tokens' write and decode attention in
 *                             one call
 * and the prefill side of the same cache:
 *   pa_prefill_attention      packed chunks of query tokens per sequence,
 *                             causal, against the same paged K/V
 * and MLA's latent cache:
 *   pa_mla_decode_attention   decode over a paged cache of latent rows, with
 *                             W_UK absorbed into the query and W_UV applied
 *                             after the softmax
 *   pa_mla_decode_step        the new latent rows written, then that decode
 * and, on the host, the bookkeeping that feeds them:
 *   pa_bm_*                   block manager: allocation in block_size units,
 *                             per-step slot_mapping / block_tables /
 *                             context_lens / cu_seqlens_q, one H2D upload
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates, frees or retains device memory and holds no state
 *     between calls except the thread-local error text and the host-memory
 *     block managers that the caller creates and destroys (pa_bm_*).
 *   - Strides and sizes are in ELEMENTS of the tensor they describe.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). Every call
 *     only enqueues work: it returns after the launch, never synchronises,
 *     never reads device memory on the host, and its launch shapes depend on
 *     host arguments only, so a call can be captured into a HIP graph.
 *   - Return value: PA_OK, or an error code with pa_last_error() describing
 *     it. On an error nothing was enqueued. Host-visible arguments are fully
 *     validated; device-resident metadata (slots, tables, lengths) cannot be
 *     checked on the host, so the kernels treat out-of-range values as
 *     documented below instead of faulting.
 *   - PA_CHECK=1 in the environment (read at every call; a test and
 *     debugging aid, not for graph capture or timing): the calls that take
 *     device-resident metadata first synchronise `stream`, copy that metadata
 *     to the host and validate it, and refuse with PA_EINVAL (nothing
 *     enqueued, pa_last_error() naming the first violation) what the kernels
 *     would otherwise skip or cannot handle: a kept token's slot outside the
 *     SWA table or the pool, two kept tokens resolving to one final slot (the
 *     writes would race), a context length outside [0, W * block_size], a
 *     used table entry outside [0, num_blocks), packed query offsets that go
 *     backwards or past the packed tokens, a chunk longer than its context.
 *   - Calls that write overlapping memory from different streams race; calls
 *     on one stream are ordered.
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 1

typedef int32_t pa_status;
enum {
  PA_OK = 0,
  PA_EINVAL = 1,       /* bad size, stride, pointer or shape relation */
  PA_EDTYPE = 2,       /* unsupported dtype or dtype combination */
  PA_EUNSUPPORTED = 3, /* valid but not implemented (e.g. head_size) */
  PA_EHIP = 4,         /* the HIP runtime reported an error at launch */
  PA_EWORKSPACE = 5,   /* workspace missing, too small or misaligned */
  PA_ENOSPACE = 6      /* block manager: not enough free blocks */
};

/* Element types. bf16 and fp32 are IEEE-style; fp8 is OCP e4m3fn (bias 7,
 * max 448, no infinities, NaN = S.1111.111), the native fp8 of gfx950. */
typedef int32_t pa_dtype;
enum { PA_BF16 = 0, PA_F32 = 2, PA_FP8_E4M3FN = 3 };

/* Text describing the last non-OK status returned on the calling thread. */
const char* pa_last_error(void);

/* PA_ABI_VERSION of the built library. */
int32_t pa_abi_version(void);

/*
 * pa_reshape_and_cache -- write token-major K (and V) into paged caches.
 *
 * Defined by: the store_kvcache Triton kernel in section 2.6 "Attention" of the
 * Qwen3-0.6B engine walkthrough page (cache layout, slot -> block/offset, the
 * skip of slot -1, source offset t*H*D + h*D + d) and reshape_and_cache_flash /
 * launch_reshape_and_cache_flash of SGLang's cache_ops.py (token strides,
 * optional second-stage SWA slot table, optional division by k/v scale before
 * the store, block stride of the cache).
 *
 * For every token t in [0, num_tokens):
 *   s = slot_mapping[t];              s < 0           -> token skipped
 *   if swa_slot_mapping:              s >= swa_len    -> skipped
 *       s = swa_slot_mapping[s];      s < 0           -> skipped
 *   s >= num_blocks*block_size                        -> skipped
 *   blk = s / block_size, off = s % block_size
 *   key_cache[blk*block_stride + (off*num_heads + h)*head_size + d]
 *       = enc(key[t*key_token_stride + h*head_size + d], k_scale)   (all h, d)
 *   and the same for value/value_cache/v_scale when value != NULL.
 * enc(x, scale):
 *   src_dtype == cache_dtype and no scale: bit copy (keeps -0 and NaN bits);
 *   otherwise y = fp32(x) / *scale (IEEE fp32 division; no division when the
 *   scale is NULL), then one round-to-nearest-even to cache_dtype:
 *     bf16: overflow -> inf; NaN -> sign | top payload bits | quiet bit;
 *     e4m3fn: |y| > 464 (rounds past 448), +-inf and NaN -> 0x7F | sign.
 *
 * Arguments
 *   key, value      [num_tokens, num_heads, head_size] with token stride
 *                   key_token_stride / value_token_stride (>= num_heads*head_size),
 *                   head stride head_size, dim stride 1. value == NULL (with
 *                   value_cache == NULL) writes K only.
 *   src_dtype       PA_BF16 or PA_F32.
 *   key_cache,      [num_blocks, block_size, num_heads, head_size], block stride
 *   value_cache     block_stride (>= block_size*num_heads*head_size), inner
 *                   [block_size, num_heads, head_size] contiguous.
 *   cache_dtype     PA_BF16, PA_F32 or PA_FP8_E4M3FN.
 *   slot_mapping    int64 [num_tokens].
 *   swa_slot_mapping  int64 [swa_len] or NULL (no remap).
 *   k_scale,v_scale device fp32 scalars; both or neither (NULL = no division).
 * Preconditions (not checkable on the host): final slots of written tokens are
 *   distinct (duplicates race: one of the writers wins per element).
 * Errors: PA_EINVAL (null pointer, negative or inconsistent sizes/strides,
 *   only one scale, value without value_cache), PA_EDTYPE, PA_EHIP.
 * num_tokens == 0 is a valid no-op.
 */
pa_status pa_reshape_and_cache(const void* key, const void* value, pa_dtype src_dtype,
                               int64_t num_tokens, int32_t num_heads, int32_t head_size,
                               int64_t key_token_stride, int64_t value_token_stride,
                               void* key_cache, void* value_cache, pa_dtype cache_dtype,
                               int64_t num_blocks, int32_t block_size, int64_t block_stride,
                               const int64_t* slot_mapping, const int64_t* swa_slot_mapping,
                               int64_t swa_len, const float* k_scale, const float* v_scale,
                               void* stream);

/*
 * pa_concat_and_cast_mla_k -- assemble MLA-style K from per-head k_nope and a
 * k_rope row shared by all heads.
 *
 * Defined by: concat_and_cast_mha_k_kernel / concat_and_cast_mha_k_triton of
 * SGLang's cache_ops.py (grid over tokens; the shape checks of the wrapper;
 * the source dtype is converted to k's dtype at the store).
 *
 *   k[t, h, d]            = cast(k_nope[t, h, d])               d < nope_dim
 *   k[t, h, nope_dim + d] = cast(k_rope[t, 0, d])               d < rope_dim
 * cast: bit copy for equal dtypes, exact widening bf16 -> fp32, and the
 * round-to-nearest-even narrowing of pa_reshape_and_cache otherwise.
 *
 * Arguments
 *   k        [num_tokens, num_heads, nope_dim + rope_dim], strides
 *            (k_stride0, k_stride1, 1); k_dtype PA_F32, PA_BF16 or PA_FP8_E4M3FN.
 *   k_nope   [num_tokens, num_heads, nope_dim], strides (nope_stride0,
 *            nope_stride1, 1); nope_dtype PA_BF16 or PA_F32.
 *   k_rope   [num_tokens, 1, rope_dim], token stride rope_stride0, dim stride 1;
 *            rope_dtype == nope_dtype.
 * Errors: PA_EINVAL (null pointers, negative sizes, strides too small for the
 *   row, overlapping rows of k), PA_EDTYPE, PA_EHIP. num_tokens == 0 is a no-op.
 */
pa_status pa_concat_and_cast_mla_k(void* k, pa_dtype k_dtype, int64_t k_stride0,
                                   int64_t k_stride1, const void* k_nope, pa_dtype nope_dtype,
                                   int64_t nope_stride0, int64_t nope_stride1,
                                   const void* k_rope, pa_dtype rope_dtype, int64_t rope_stride0,
                                   int64_t num_tokens, int32_t num_heads, int32_t nope_dim,
                                   int32_t rope_dim, void* stream);

/*
 * pa_concat_and_cache_mla_k -- the MLA K assembly written straight into the
 * paged cache: per-head k_nope ++ shared k_rope, cast, scattered through the
 * slot mapping, with no K intermediate in device memory.
 *
 * Defined by: the composition of concat_and_cast_mha_k and
 * reshape_and_cache_flash (K only) of SGLang's cache_ops.py, the two ops the
 * hot path runs back to back for an MLA-style K. The result is bit-identical
 * to pa_concat_and_cast_mla_k into an fp32 K followed by
 * pa_reshape_and_cache(K, NULL, key_cache, NULL, ..., slot_mapping,
 * swa_slot_mapping, swa_len, k_scale, NULL): each element is widened exactly
 * to fp32, divided by *k_scale when k_scale is given, and rounded once to the
 * cache type; slot resolution and skips are those of pa_reshape_and_cache.
 *
 * Arguments
 *   k_nope   [num_tokens, num_heads, nope_dim], strides (nope_stride0,
 *            nope_stride1, 1); src_dtype PA_BF16 or PA_F32.
 *   k_rope   [num_tokens, 1, rope_dim], token stride rope_stride0; src_dtype.
 *   key_cache [num_blocks, block_size, num_heads, nope_dim + rope_dim], block
 *            stride block_stride, inner part contiguous; cache_dtype PA_BF16,
 *            PA_F32 or PA_FP8_E4M3FN.
 *   slot_mapping, swa_slot_mapping, swa_len, k_scale: as pa_reshape_and_cache.
 * Supported: nope_dim and rope_dim multiples of 8, (nope_dim + rope_dim) <= 2048;
 *   16-byte aligned source rows, cache blocks aligned to 16 bytes (8 for fp8).
 * Errors: PA_EINVAL, PA_EDTYPE, PA_EUNSUPPORTED, PA_EHIP. num_tokens == 0 or
 * num_blocks == 0 is a valid no-op.
 */
pa_status pa_concat_and_cache_mla_k(const void* k_nope, pa_dtype src_dtype, int64_t nope_stride0,
                                    int64_t nope_stride1, const void* k_rope, int64_t rope_stride0,
                                    int64_t num_tokens, int32_t num_heads, int32_t nope_dim,
                                    int32_t rope_dim, void* key_cache, pa_dtype cache_dtype,
                                    int64_t num_blocks, int32_t block_size, int64_t block_stride,
                                    const int64_t* slot_mapping, const int64_t* swa_slot_mapping,
                                    int64_t swa_len, const float* k_scale, void* stream);

/*
 * pa_decode_attention_workspace_size -- bytes of device workspace that
 * pa_decode_attention needs for these sizes (a pure function of its
 * arguments; 0 is never returned for valid sizes). Returns 0 and sets
 * pa_last_error() for invalid sizes.
 */
size_t pa_decode_attention_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_size,
                                          int32_t max_blocks_per_seq, int32_t block_size);

/*
 * pa_decode_attention -- single-token paged decode attention with GQA.
 *
 * Defined by: section 2.6 "Attention" of the Qwen3-0.6B engine walkthrough
 * page (the decode attention kernel reads K/V back along physical blocks
 * through block_tables) and the PagedAttention principle page (GQA: H_Q is an
 * integer multiple of H_KV; decode writes the new token's K/V before
 * attention; a block is [block_size, H_KV, d_h]; blocks are physically
 * scattered and ordered only by a table). Attention itself is the standard
 * scaled-dot-product softmax; groups are contiguous (q head h reads kv head
 * h / (num_q_heads / num_kv_heads)).
 *
 * For sequence b with n = clamp(context_lens[b], 0, max_blocks_per_seq*block_size)
 * and q head h (g = h / G):
 *   row(p)   = block_tables[b*max_blocks_per_seq + p/block_size], offset p%block_size
 *   s_p      = softmax_scale * sum_d q[b,h,d] * (K[row(p), p%bs, g, d] * k_scale)
 *   out[b,h] = sum_p softmax(s)_p * (V[row(p), p%bs, g, :] * v_scale)    (p < n)
 * n == 0 writes zeros. A table entry outside [0, num_blocks) removes its
 * positions from the softmax instead of being dereferenced.
 *
 * Arguments
 *   out      [num_seqs, num_q_heads, head_size], sequence stride out_seq_stride;
 *            out_dtype PA_BF16 or PA_F32 (round to nearest even from fp32).
 *   q        [num_seqs, num_q_heads, head_size], sequence stride q_seq_stride;
 *            q_dtype PA_BF16.
 *   key_cache, value_cache  [num_blocks, block_size, num_kv_heads, head_size],
 *            block stride block_stride, inner part contiguous; cache_dtype
 *            PA_BF16 or PA_FP8_E4M3FN.
 *   block_tables  int32 [num_seqs, max_blocks_per_seq], row-major, device.
 *   context_lens  int32 [num_seqs], device.
 *   k_scale, v_scale  device fp32 scalars or NULL (= 1.0).
 *   workspace, workspace_bytes  device scratch of at least
 *            pa_decode_attention_workspace_size(...) bytes, 256-byte aligned;
 *            it receives the per-split partial results, so its contents on
 *            entry do not matter. Concurrent calls must not share it.
 * Supported: head_size in {64, 128, 256}; num_q_heads % num_kv_heads == 0 with
 *   num_q_heads / num_kv_heads in {1, 2, 4, 8}; block_size a multiple of
 *   64 / (head_size / 8).
 * Errors: PA_EINVAL, PA_EDTYPE, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EHIP.
 * num_seqs == 0 is a valid no-op.
 */
pa_status pa_decode_attention(void* out, pa_dtype out_dtype, int64_t out_seq_stride,
                              const void* q, pa_dtype q_dtype, int64_t q_seq_stride,
                              const void* key_cache, const void* value_cache,
                              pa_dtype cache_dtype, int64_t num_blocks, int32_t block_size,
                              int64_t block_stride, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_size, float softmax_scale, const float* k_scale,
                              const float* v_scale, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * pa_decode_attention_noalloc -- pa_decode_attention for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments and results as
 * pa_decode_attention without the workspace: the per-split partial results go
 * to a fixed device array of pa_decode_attention_noalloc_max_workspace()
 * bytes (64 MiB) inside the library, one copy per GPU, held until the process
 * ends. The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine); its first call on a device looks up that device's copy
 * of the array (hipGetSymbolAddress).
 * Every call on one GPU shares that GPU's array, and the array keeps the last
 * call's contents (the kernels need nothing from it on entry): calls that
 * overlap in time on one GPU (different streams, or different host threads
 * without ordering) race and must not be made.
 * Errors: those of pa_decode_attention; PA_EWORKSPACE when
 * pa_decode_attention_workspace_size() of these sizes exceeds the array.
 */
size_t pa_decode_attention_noalloc_max_workspace(void);
pa_status pa_decode_attention_noalloc(void* out, pa_dtype out_dtype, int64_t out_seq_stride,
                                      const void* q, pa_dtype q_dtype, int64_t q_seq_stride,
                                      const void* key_cache, const void* value_cache,
                                      pa_dtype cache_dtype, int64_t num_blocks,
                                      int32_t block_size, int64_t block_stride,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_size, float softmax_scale,
                                      const float* k_scale, const float* v_scale, void* stream);

/*
 * pa_decode_step -- one decode step in one call: the new tokens' K/V are
 * written into the paged caches and single-token decode attention runs over
 * the contexts that now include them. Launch shapes depend on host arguments
 * only (graph-capturable; no allocation, no host synchronisation).
 *
 * Defined by: "PagedAttention principle" page, autoregressive dataflow section
 * (a decode step computes the new token's q/k/v, writes the KV cache, then
 * computes attention), i.e. pa_reshape_and_cache followed by
 * pa_decode_attention. The result equals that sequence of calls:
 *   pa_reshape_and_cache(new_k, new_v, new_dtype, num_seqs, num_kv_heads,
 *       head_size, new_k_stride, new_v_stride, key_cache, value_cache,
 *       cache_dtype, num_blocks, block_size, block_stride, new_slots, NULL, 0,
 *       k_scale, v_scale, stream);
 *   pa_decode_attention(out, ..., context_lens, ..., workspace, ...);
 * where context_lens[b] already counts the new token (position
 * context_lens[b] - 1). Every argument is checked before anything is
 * enqueued, so an error leaves no work queued. For the persistent kernel's
 * shapes (block_size a multiple of 16, head_size <= 128) the call launches
 * two kernels: the attention over the cached positions, which leaves out
 * position ctx-1 when new_slots[b] is that position's slot, and the merge
 * pass, which takes the new token in from new_k / new_v as the cache write
 * encodes it and then writes its row into new_slots[b]. The caches end up
 * bit-identical to the two separate calls; the output differs from theirs
 * only in the order of fp32 sums. Other shapes enqueue the cache write, then
 * the attention.
 * Precondition (no check is possible on the host): new_slots[b], when it is
 * written, is not the slot of any other position that some sequence's
 * context reads in this call.
 *
 * Arguments
 *   new_k, new_v  [num_seqs, num_kv_heads, head_size], sequence strides
 *            new_k_stride / new_v_stride (elements); new_dtype PA_BF16.
 *   new_slots  int64 [num_seqs], device: each new token's cache slot
 *            (negative or outside the pool = not written, as in
 *            pa_reshape_and_cache).
 *   k_scale, v_scale  both or neither: the write divides by them, the
 *            attention multiplies by them.
 *   everything else as pa_decode_attention (same workspace size).
 * Supported: every shape and cache type of pa_decode_attention.
 * Errors: PA_EINVAL, PA_EDTYPE, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EHIP.
 */
pa_status pa_decode_step(const void* new_k, const void* new_v, pa_dtype new_dtype,
                         int64_t new_k_stride, int64_t new_v_stride, const int64_t* new_slots,
                         void* out, pa_dtype out_dtype, int64_t out_seq_stride, const void* q,
                         pa_dtype q_dtype, int64_t q_seq_stride, void* key_cache,
                         void* value_cache, pa_dtype cache_dtype, int64_t num_blocks,
                         int32_t block_size, int64_t block_stride, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_size, float softmax_scale, const float* k_scale,
                         const float* v_scale, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * pa_prefill_attention -- chunked-prefill (variable-length, causal) paged
 * attention with GQA: many query tokens per sequence against the sequence's
 * paged K/V, the other half of an engine's attention next to decode.
 *
 * Defined by: Qwen3-0.6B engine walkthrough page, section 2.4 (prefill queries
 * are packed token-major and delimited by cu_seqlens_q, the prefix sums of
 * the per-sequence query counts) and section 2.6 (the variable-length flash
 * path of prefill); "PagedAttention principle" page, autoregressive dataflow
 * section (prefill attends causally over the prompt while caching its K/V).
 *
 * Sequence b owns packed query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1,
 * n_b of them: the LAST n_b positions of its context (their K/V are already
 * in the cache, written by pa_reshape_and_cache). With
 * L = clamp(context_lens[b], 0, max_blocks_per_seq*block_size), query i sits
 * at position p = L - n_b + i and, for q head h (g = h / G),
 *   out[row, h] = sum_{j<=p} softmax_j(softmax_scale * q[row,h,:].K^[j,g,:]) V^[j,g,:]
 * with K^ = K * k_scale, V^ = V * v_scale, positions gathered through
 * block_tables[b] exactly as in pa_decode_attention (an entry outside
 * [0, num_blocks) removes its positions). A query with p < 0 (n_b > L) has no
 * key and gets zeros. n_b == 1 is the decode step of pa_decode_attention.
 *
 * Arguments
 *   out      [num_tokens, num_q_heads, head_size], token stride
 *            out_token_stride; out_dtype PA_BF16 or PA_F32.
 *   q        [num_tokens, num_q_heads, head_size], token stride q_token_stride;
 *            q_dtype PA_BF16.
 *   cu_seqlens_q  int32 [num_seqs + 1], device: 0 = cu[0] <= cu[1] <= ... <=
 *            cu[num_seqs] = num_tokens (values are clamped into [0, num_tokens]
 *            for memory safety; rows no sequence owns are not written).
 *   key_cache, value_cache, block_tables, context_lens, k_scale, v_scale: as
 *            for pa_decode_attention; cache_dtype PA_BF16 or PA_FP8_E4M3FN
 *            (fp8 values are dequantised by multiplying with the scales).
 * No workspace: each query row's softmax is completed inside one workgroup.
 * Supported: head_size in {64, 128, 256}; num_q_heads / num_kv_heads in
 *   {1, 2, 4, 8}; block_size a multiple of 16.
 * Errors: PA_EINVAL, PA_EDTYPE, PA_EUNSUPPORTED, PA_EHIP. num_seqs == 0 or
 * num_tokens == 0 is a valid no-op.
 */
pa_status pa_prefill_attention(void* out, pa_dtype out_dtype, int64_t out_token_stride,
                               const void* q, pa_dtype q_dtype, int64_t q_token_stride,
                               int64_t num_tokens, const int32_t* cu_seqlens_q,
                               const void* key_cache, const void* value_cache,
                               pa_dtype cache_dtype, int64_t num_blocks, int32_t block_size,
                               int64_t block_stride, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_size, float softmax_scale, const float* k_scale,
                               const float* v_scale, void* stream);

/*
 * pa_hbm_copy -- streaming device-to-device copy of `bytes` bytes
 * (measurement utility, not part of the cache path): the reference kernel
 * against which achieved HBM bandwidth and profiler byte counters are
 * calibrated. dst and src must be 16-byte aligned and must not overlap.
 * Errors: PA_EINVAL, PA_EHIP.
 */
pa_status pa_hbm_copy(void* dst, const void* src, size_t bytes, void* stream);

/*
 * pa_hbm_read -- streaming read of `bytes` bytes at `src` (measurement utility,
 * not part of the cache path): the read-only bandwidth reference for the decode
 * kernels, which read far more than they write. `sink` is caller-owned device
 * memory of PA_HBM_READ_SINK_UNITS 16-byte units; a call with bytes > 0
 * overwrites all of them with partial XOR folds of src's 16-byte units, whose
 * XOR is the XOR of every unit of src (so a check proves every byte was read);
 * bytes == 0 enqueues nothing. bytes must be a multiple of 16; src and sink
 * 16-byte aligned. Errors: PA_EINVAL, PA_EHIP.
 */
#define PA_HBM_READ_SINK_UNITS 2048
pa_status pa_hbm_read(const void* src, size_t bytes, void* sink, void* stream);

/*
 * pa_mla_decode_workspace_size -- bytes of device workspace
 * pa_mla_decode_attention needs for these sizes (256-byte aligned); 0 with
 * pa_last_error() set if the shape is unsupported. Pure function.
 */
size_t pa_mla_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t qk_nope_dim,
                                    int32_t rope_dim, int32_t kv_lora_rank, int32_t v_dim,
                                    int32_t max_blocks_per_seq, int32_t block_size);

/*
 * pa_mla_decode_attention -- single-token decode attention of MLA over a
 * paged cache of latent rows.
 *
 * Defined by: "PagedAttention principle" page, MLA paragraphs of the GQA/MLA
 * shapes section: per token MLA caches the latent c = x W_DKV (kv_lora_rank
 * values) instead of K and V; head h's key and value are (c W_UK) and (c W_UV)
 * split per head; the q.k dimension also carries a RoPE part that v lacks.
 * Each cached row here is c followed by rope_dim values of a RoPE key shared
 * by all heads (the row pa_concat_and_cache_mla_k writes with num_heads = 1,
 * nope_dim = kv_lora_rank). For sequence b and head h, over positions p <
 * context_lens[b] read through block_tables (clamping and table-entry rule as
 * pa_decode_attention):
 *   s_p = softmax_scale * (q_nope[b,h] . (c_p W_UK)[h] + q_rope[b,h] . k_r,p)
 *   out[b,h,:] = sum_p softmax(s)_p (c_p W_UV)[h]
 * computed with the products re-associated: W_UK is applied to the query
 * once, the softmax runs over the latent rows, and W_UV is applied to the
 * weighted latent sum, so each cached row is read once and never expanded.
 * Internally the absorbed query and the probabilities are carried as bf16
 * hi + lo pairs on the matrix cores (about 16 bits beyond bf16), everything
 * else in fp32.
 *
 * Arguments
 *   out      [num_seqs, num_heads, v_dim], sequence stride out_seq_stride;
 *            out_dtype PA_BF16 or PA_F32.
 *   q_nope   [num_seqs, num_heads, qk_nope_dim], sequence stride
 *            q_nope_seq_stride, 16-byte aligned per sequence; q_rope [num_seqs, num_heads, rope_dim],
 *            sequence stride q_rope_seq_stride (unused when rope_dim = 0);
 *            q_dtype PA_BF16.
 *   w_uk     [kv_lora_rank, num_heads * qk_nope_dim] row-major (c W_UK gives
 *            the keys of all heads, head-major); w_uv [kv_lora_rank,
 *            num_heads * v_dim] likewise; w_dtype PA_BF16; 16-byte aligned.
 *   latent_cache [num_blocks, block_size, kv_lora_rank + rope_dim], block
 *            stride block_stride (elements); cache_dtype PA_BF16.
 *   block_tables, max_blocks_per_seq, context_lens, num_seqs: as
 *            pa_decode_attention.
 *   workspace  >= pa_mla_decode_workspace_size(...) bytes, 256-byte aligned;
 *            contents are scratch.
 * Supported: num_heads 16 (one tensor-parallel shard of a larger model's
 *   heads per call), kv_lora_rank 512, rope_dim 0 or 64, qk_nope_dim a
 *   multiple of 8 up to 256, v_dim = 8 * a divisor of 256.
 * Errors: PA_EINVAL, PA_EDTYPE, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EHIP.
 * num_seqs == 0 is a valid no-op. The attention kernel's waves hand work to
 * each other through bounded waits; should one ever run past its bound (it
 * does not when every wave of a workgroup runs), the call ends instead of
 * hanging and every output of the call is NaN.
 */
pa_status pa_mla_decode_attention(void* out, pa_dtype out_dtype, int64_t out_seq_stride,
                                  const void* q_nope, int64_t q_nope_seq_stride,
                                  const void* q_rope, int64_t q_rope_seq_stride, pa_dtype q_dtype,
                                  const void* w_uk, const void* w_uv, pa_dtype w_dtype,
                                  const void* latent_cache, pa_dtype cache_dtype,
                                  int64_t num_blocks, int32_t block_size, int64_t block_stride,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t num_heads, int32_t qk_nope_dim, int32_t rope_dim,
                                  int32_t kv_lora_rank, int32_t v_dim, float softmax_scale,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_mla_decode_step -- one decode step over the latent cache: the batch's new
 * latent rows written, then pa_mla_decode_attention over the cache that holds
 * them.
 *
 * Defined by: "PagedAttention principle" page, the decode dataflow section (each
 * step stores the new token's cache entry through its slot, then attends over
 * the sequence's blocks) with the MLA paragraphs of the GQA/MLA shapes section
 * (what is stored per token is the latent c and the shared RoPE key). Sequence
 * b's row c = new_c[b] (kv_lora_rank values) followed by new_rope[b] (rope_dim
 * values) goes to slot new_slots[b] of latent_cache (block slot / block_size,
 * offset slot % block_size), exactly as pa_concat_and_cache_mla_k with
 * num_heads = 1 writes it; a negative slot, or one past num_blocks *
 * block_size, writes nothing. The attention then reads the cache with the
 * rows in place (a new position is normally the last, context_lens[b] - 1).
 * The rows are written by the launch that also absorbs the query, so the step
 * takes three kernels, as the attention alone.
 *
 * Arguments
 *   new_c    [num_seqs, kv_lora_rank], row stride new_c_stride (elements),
 *            16-byte aligned per row; new_rope [num_seqs, rope_dim], row
 *            stride new_rope_stride, 16-byte aligned per row (unused when
 *            rope_dim = 0); new_dtype PA_BF16 (the cache's type: a copy).
 *   new_slots [num_seqs] int64, device; two kept rows must not share a slot.
 *   the rest: as pa_mla_decode_attention, with latent_cache writable.
 * Errors: as pa_mla_decode_attention; nothing is written or launched when a
 * call returns an error.
 */
pa_status pa_mla_decode_step(const void* new_c, int64_t new_c_stride, const void* new_rope,
                             int64_t new_rope_stride, pa_dtype new_dtype, const int64_t* new_slots,
                             void* out, pa_dtype out_dtype, int64_t out_seq_stride,
                             const void* q_nope, int64_t q_nope_seq_stride,
                             const void* q_rope, int64_t q_rope_seq_stride, pa_dtype q_dtype,
                             const void* w_uk, const void* w_uv, pa_dtype w_dtype,
                             void* latent_cache, pa_dtype cache_dtype, int64_t num_blocks,
                             int32_t block_size, int64_t block_stride, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t num_seqs, int32_t num_heads, int32_t qk_nope_dim,
                             int32_t rope_dim, int32_t kv_lora_rank, int32_t v_dim,
                             float softmax_scale, void* workspace, size_t workspace_bytes,
                             void* stream);

/* ------------------------------------------------------------------------
 * Block manager (host side).
 *
 * Defined by: "PagedAttention principle" page, paged attention principle
 * section -- memory is handed out in blocks of block_size token slots, so a
 * request of n tokens holds ceil(n / block_size) blocks and wastes less than
 * one; a sequence's blocks need not be adjacent, a table keeps their order;
 * the host knows every request's blocks and copies the table to the device
 * before the launch; and the design must stay usable under graph capture
 * (fixed shapes, no data-dependent host branching in the captured work).
 * The slot of a position is the Qwen3-0.6B engine walkthrough page's
 * (section 2.6): slot = block * block_size + offset.
 *
 * Sequences are ids 0..max_seqs-1. A sequence's length is the number of
 * token positions it has been given; it holds exactly ceil(length /
 * block_size) blocks, listed in position order in its table. A step grows a
 * set of sequences by some tokens each (a prefill chunk, or one token per
 * sequence in decode) and produces that step's metadata: the slot of every
 * new token, the block table, context length (the new length) and packed
 * query offsets of every listed sequence, in one host blob laid out by
 * pa_bm_layout_of; pa_bm_upload copies the blob to the device in one copy,
 * after which the device pointers base + offset are the kernels' arguments.
 *
 * Allocation order (deterministic): free blocks form a stack that starts as
 * 0, 1, ..., num_blocks-1 from the top; a step takes new blocks from the top,
 * sequence by sequence in the order listed, positions in increasing order;
 * pa_bm_release pushes a sequence's blocks back so that its first block is
 * on top. A manager is not thread-safe; it lives in host memory only.
 * ------------------------------------------------------------------------ */
typedef struct pa_block_manager pa_block_manager;

/* Byte offsets of the step blob's arrays (each 256-byte aligned):
 *   context_lens  int32 [max_step_seqs]
 *   cu_seqlens_q  int32 [max_step_seqs + 1]
 *   slot_mapping  int64 [max_step_tokens]
 *   block_tables  int32 [max_step_seqs, max_blocks_per_seq]  (last)
 * bytes = the whole blob. */
typedef struct {
  int64_t context_lens;
  int64_t cu_seqlens_q;
  int64_t slot_mapping;
  int64_t block_tables;
  int64_t bytes;
} pa_bm_layout;

/*
 * pa_bm_create -- a manager of num_blocks blocks of block_size slots for up
 * to max_seqs sequences of at most max_blocks_per_seq blocks each; a step
 * lists at most max_step_seqs sequences and adds at most max_step_tokens
 * tokens. All sizes > 0; num_blocks and max_blocks_per_seq * block_size fit
 * int32. *out receives the manager (NULL on error).
 * Errors: PA_EINVAL.
 */
pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, int32_t max_seqs,
                       int32_t max_blocks_per_seq, int32_t max_step_seqs,
                       int64_t max_step_tokens, pa_block_manager** out);

/* Frees the manager's host memory (NULL is a no-op). */
void pa_bm_destroy(pa_block_manager* bm);

/* The step blob's layout. Errors: PA_EINVAL (NULL argument). */
pa_status pa_bm_layout_of(const pa_block_manager* bm, pa_bm_layout* out);

/* Free blocks now; -1 for a NULL manager. */
int64_t pa_bm_free_blocks(const pa_block_manager* bm);

/* Length of sequence `seq`; -1 for a bad id or NULL manager. */
int64_t pa_bm_seq_len(const pa_block_manager* bm, int32_t seq);

/* Copies sequence `seq`'s block table (position order) into blocks[0..);
 * returns the number of blocks, or -1 for a bad id, a NULL pointer or a
 * capacity below that number. */
int32_t pa_bm_seq_table(const pa_block_manager* bm, int32_t seq, int32_t* blocks,
                        int32_t capacity);

/* Returns every block of sequence `seq` to the free stack; its length
 * becomes 0. Releasing an empty sequence is a no-op.
 * Errors: PA_EINVAL (bad id, NULL manager). */
pa_status pa_bm_release(pa_block_manager* bm, int32_t seq);

/*
 * pa_bm_plan_step -- grow sequence seqs[i] by num_new[i] tokens (i <
 * num_seqs) and write the step blob into host_meta:
 *   context_lens[i]  = the new length (the chunk of sequence i is its last
 *                      num_new[i] positions);
 *   cu_seqlens_q[i]  = num_new[0] + ... + num_new[i-1] (i <= num_seqs);
 *   slot_mapping[cu_seqlens_q[i] + j] = slot of position old_len_i + j;
 *   block_tables[i, k] = the sequence's k-th block, -1 past its last block.
 * Rows num_seqs..pad_seqs-1 are filled as empty sequences (length 0,
 * cu_seqlens_q = the total, table all -1) and slot_mapping entries
 * total..pad_tokens-1 with -1, so a caller can launch every step with the
 * fixed sizes (pad_seqs, pad_tokens) -- the padding is a no-op for the
 * kernels. *num_tokens receives the total of num_new (may be NULL).
 * Either the whole step is applied or, on any error, nothing changes.
 * Arguments: seqs distinct ids; num_new[i] >= 0; num_seqs <= pad_seqs <=
 *   max_step_seqs; total <= pad_tokens <= max_step_tokens; no sequence may
 *   exceed max_blocks_per_seq blocks; host_meta >= layout bytes, 8-byte
 *   aligned (pinned memory if it is to be uploaded asynchronously).
 * Errors: PA_EINVAL, PA_ENOSPACE (fewer free blocks than the step needs).
 */
pa_status pa_bm_plan_step(pa_block_manager* bm, const int32_t* seqs, const int32_t* num_new,
                          int32_t num_seqs, int32_t pad_seqs, int64_t pad_tokens,
                          void* host_meta, int64_t host_meta_bytes, int64_t* num_tokens);

/*
 * pa_bm_upload -- one asynchronous host-to-device copy of the step blob's
 * used part (everything before block_tables, then pad_seqs table rows) from
 * host_meta to device_meta (a device buffer of layout bytes, 256-byte
 * aligned) on `stream`. With pinned host memory and a fixed pad_seqs the copy
 * can be captured into a HIP graph; the host must not rewrite host_meta
 * until the copy has executed.
 * Errors: PA_EINVAL, PA_EHIP.
 */
pa_status pa_bm_upload(const pa_block_manager* bm, const void* host_meta, void* device_meta,
                       int32_t pad_seqs, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
