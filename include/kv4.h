/*
 * kv4.h -- C ABI of libkv4: INT4 per-token-head KV cache with a randomized
 * Hadamard rotation, for AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [PR40835] vLLM PR #40835, "[Feature] Triton INT4 per-token-head KV cache
 *             quantization" -- review thread: float32 scale caches of shape
 *             [num_blocks, block_size, num_kv_heads], uint8 int4 cache,
 *             slot_mapping [num_tokens], query_start_loc / seq_lens metadata,
 *             prefill and decode served by one unified attention entry point.
 *   [PR56198] runguoli.com, "vLLM -- Attention Kernels & KV Cache
 *             Quantization", section "PR #56198 -- Support int4_per_token_head
 *             on non-power-of-two head sizes": head_size d = b * n with b the
 *             largest power-of-two divisor; H_b applied block-diagonally; the
 *             read path compensates by b; every head size is accepted.
 *   [PR62881] vLLM PR #62881, "[Bugfix][Test] Rotate KV into RHT domain in the
 *             INT4 unified attn test", Details / Root cause and Fix: the write
 *             path stores K_s = H.D.k (rounded through bf16); the read path
 *             rotates q' = H.D.q, scales logits by softmax_scale / b and maps
 *             the output back with D.H(.)/b.
 *
 * Numerics fixed where the pages are silent:
 *   D      sign i (0 <= i < head_size) is -1 iff bit 63 of the (i+1)-th
 *          SplitMix64 output from state sign_seed is set; one D shared by K,
 *          V, Q, every head and token.
 *   H_b    unnormalized Sylvester-order Walsh-Hadamard matrix, applied to the
 *          contiguous chunks [j*b, (j+1)*b) of each head vector.
 *   write  x (bf16) -> sign flip -> radix-2 butterflies in float32 with strides
 *          1, 2, ..., b/2 in that order -> one round-to-nearest-even to bf16 ->
 *          scale = absmax / 7 (IEEE float32 division) -> code =
 *          clamp(rint_half_even(y / scale), -8, 7) -> two's-complement nibbles,
 *          element 2j in the low nibble of byte j. absmax == 0 stores scale 0
 *          and zero codes.
 *   read   query i of a sequence with query_len q and seq_len L is at position
 *          L - q + i and attends to keys 0 .. L - q + i (causal). GQA: query
 *          head h reads kv head h / (num_q_heads / num_kv_heads).
 *
 * Conventions shared by every entry point:
 *   - All tensors are caller-owned device buffers (hipMalloc / torch); the
 *     library never allocates, frees or synchronizes.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the legacy default
 *     stream) and is asynchronous: a KV4_OK return means the arguments were
 *     valid and the launches were queued.
 *   - Arguments are validated on the host before any launch. On failure the
 *     function returns a nonzero kv4_status, launches nothing, and
 *     kv4_last_error() (thread-local) describes the problem.
 *   - Device data that the host cannot see (slot ids, block ids, lengths) is
 *     range-checked inside the kernels: an out-of-range slot is skipped, an
 *     out-of-range page id contributes nothing, lengths are clamped to the
 *     page-table capacity. Kernels never read or write outside the buffers
 *     whose sizes the arguments describe.
 *   - Pointers must be 16-byte aligned (the cache rows are read with 16-byte
 *     vector loads; vLLM PR #62113 aligned per-token-head KV slots to 16 bytes
 *     for the same reason).
 *   - head_size: a multiple of 8 in [8, 256]; b must equal the largest power
 *     of two dividing head_size ([PR56198]), or be 0 to let the library take
 *     that value; anything else is KV4_EINVAL.
 *   - block_size (tokens per page) may be any value in [1, 4096]; the
 *     matrix-core attention kernel serves powers of two >= 16 and the vector
 *     kernel every other size, with the same results.
 *   - Every entry point that does work returns a kv4_status; the
 *     *_workspace_size queries return a byte count (0 with an error message
 *     for invalid sizes).
 */
#ifndef KV4_H_
#define KV4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KV4_OK = 0,
  KV4_EINVAL = 1,        /* invalid argument (shape, pointer, alignment)      */
  KV4_EUNSUPPORTED = 2,  /* valid but not supported by this library           */
  KV4_EHIP = 3,          /* a HIP runtime call or kernel launch failed        */
  KV4_EWORKSPACE = 4     /* workspace missing or smaller than required        */
} kv4_status;

/*
 * kv4_rht_write -- the write path, reshape_and_cache_int4 ([PR62881] Root
 * cause; block-diagonal H_b per [PR56198]; scale cache shapes per [PR40835]).
 *
 * For every token t with slot s = slot_mapping[t] in [0, num_blocks*block_size)
 * and every kv head h, rotates key[t, h, :] and value[t, h, :] (K_s = H.D.k),
 * rounds through bf16, quantizes to int4 with one float32 scale, and stores
 *   key_cache  [s / block_size, s % block_size, h, :]  (head_size/2 bytes)
 *   k_scale_cache[s / block_size, s % block_size, h]   (float32)
 * and likewise for value. Slots < 0 or >= num_blocks*block_size are skipped.
 * Duplicate slots in one call race (the stored bytes are then unspecified);
 * with the environment variable KV4_CHECK_SLOTS=1 every write entry point
 * copies the slot map to the host first (the call then waits for the
 * stream) and returns KV4_EINVAL, before any launch, if a slot in
 * [0, num_blocks * block_size) appears twice.
 *
 *   key, value          bf16 [num_tokens, num_kv_heads, head_size]; rows of
 *                       consecutive tokens are key_token_stride /
 *                       value_token_stride elements apart (>= nkv*head_size,
 *                       multiple of 8); heads are contiguous within a row.
 *   key_cache,
 *   value_cache         uint8 [num_blocks, block_size, num_kv_heads, head_size/2]
 *   k_scale_cache,
 *   v_scale_cache       float32 [num_blocks, block_size, num_kv_heads]
 *   slot_mapping        int64 [num_tokens]
 *   sign_seed           seed of D (see above)
 * num_tokens == 0 is a valid no-op.
 */
kv4_status kv4_rht_write(const void* key, const void* value,
                         int64_t key_token_stride, int64_t value_token_stride,
                         void* key_cache, void* value_cache,
                         float* k_scale_cache, float* v_scale_cache,
                         const int64_t* slot_mapping, int64_t num_tokens,
                         int32_t num_kv_heads, int32_t head_size, int32_t b,
                         int32_t block_size, int64_t num_blocks,
                         uint64_t sign_seed, void* stream);

/*
 * kv4_paged_attention_workspace_size -- bytes of device workspace that
 * kv4_paged_attention needs for these sizes (split-KV partial results and
 * their merge). Depends only on the host-known sizes listed. Returns 0 for
 * invalid sizes (kv4_last_error() then says why) -- callers should treat 0
 * with num_q_tokens > 0 as an error.
 */
size_t kv4_paged_attention_workspace_size(int64_t num_q_tokens, int32_t num_seqs,
                                          int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_size, int32_t max_query_len,
                                          int32_t max_seq_len);

/*
 * kv4_paged_attention -- the read path, unified_attention_int4 ([PR62881]
 * Root cause; compensation by b per [PR56198]; metadata per [PR40835]).
 * Prefill, decode and mixed batches in one call, causal.
 *
 * For sequence s with query rows query_start_loc[s] .. query_start_loc[s+1]
 * and total KV length seq_lens[s] (including the new tokens, already written
 * with kv4_rht_write), computes for each query head
 *   q' = H.D.q,  logit_j = k_scale_j * (q' . code_K_j) * softmax_scale / b,
 *   o' = sum_j softmax(logit)_j * v_scale_j * code_V_j,  out = D.H.o' / b,
 * reading K/V pages through block_table, and writes out as bf16 (one
 * round-to-nearest-even of the float32 result).
 *
 *   query               bf16 [num_q_tokens, num_q_heads, head_size], token
 *                       rows query_token_stride elements apart (multiple of 8)
 *   key_cache, ...      as written by kv4_rht_write; num_blocks pages
 *   block_table         int32 [num_seqs, max_blocks_per_seq], page ids
 *   seq_lens            int32 [num_seqs]        (device)
 *   query_start_loc     int32 [num_seqs + 1]    (device), non-decreasing,
 *                       query_start_loc[num_seqs] == num_q_tokens
 *   max_query_len,
 *   max_seq_len         host-side upper bounds of the device lengths; rows and
 *                       keys beyond them are not computed
 *   softmax_scale       the model's scale (e.g. head_size^-0.5); the kernels
 *                       multiply logits by softmax_scale / b
 *   out                 bf16 [num_q_tokens, num_q_heads, head_size], contiguous
 *   workspace           device buffer of at least
 *                       kv4_paged_attention_workspace_size(...) bytes; its
 *                       contents need no initialization and are clobbered.
 *                       Two calls in flight must not share a workspace.
 * A query row whose causal window is empty (seq_len < query_len) gets zeros.
 *
 * The launch plan (matrix-core or vector path, KV split size, kv heads per
 * matrix-core wave) is chosen on the host from the sizes above. Environment
 * variables, read at each call, override it for testing and tuning:
 * KV4_FORCE_PATH=valu|mfma, KV4_SPLIT_TOKENS=<tokens per split>,
 * KV4_MFMA_HPW=1|2|4 (lowered where the shape does not allow it),
 * KV4_STREAMK=0 (split-KV instead of the stream-K decode schedule),
 * KV4_SK_GRID=<stream-K workgroups at most>, KV4_MFMA_RB=1 (one 16-row block
 * per wave), KV4_REDUCE_ROWS=0|1 (merge form), KV4_FUSED_PLAN=0 (separate
 * plan kernel), KV4_NT=0|1 (non-temporal K/V code loads, where a kernel is
 * built with them), KV4_PREFILL=0|1 (int4, head size 128: the chunked-prefill
 * kernel never / wherever the shape allows; by default where long chunks
 * carry the batch), KV4_FORK=0 (see below). Results agree within the rounding
 * of the float32 accumulation order; KV4_NT, KV4_FUSED_PLAN and KV4_FORK
 * leave them bit-identical.
 * With the prefill kernel, the other sequences' launches run on a stream the
 * library owns (one per device), forked from `stream` with an event before
 * them and joined back into it with an event after them, so that they fill
 * the CUs the prefill workgroups leave; the call stays ordered on `stream`
 * (KV4_FORK=0 runs everything on `stream`). Calls from several threads on
 * one device take turns on that stream.
 * kv4_paged_attention_workspace_size reads the same variables: query it with
 * the same environment the call will see.
 */
kv4_status kv4_paged_attention(const void* query, int64_t query_token_stride,
                               const void* key_cache, const void* value_cache,
                               const float* k_scale_cache, const float* v_scale_cache,
                               int64_t num_blocks,
                               const int32_t* block_table, int32_t max_blocks_per_seq,
                               const int32_t* seq_lens, const int32_t* query_start_loc,
                               int32_t num_seqs, int64_t num_q_tokens,
                               int32_t max_query_len, int32_t max_seq_len,
                               int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_size, int32_t b, int32_t block_size,
                               uint64_t sign_seed, float softmax_scale,
                               void* out, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * kv4_paged_attention_noalloc -- kv4_paged_attention for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * must not call hipMalloc, harnesses that forbid it). Same arguments, results
 * and errors, without the workspace: the split partials live in a static
 * device array of KV4_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 * held from the library's first use on that GPU until the process ends. The
 * call allocates and frees nothing. A batch whose plan needs more scratch than
 * that returns KV4_EWORKSPACE before any launch (the single-token decode
 * batches of the Phi-3, Llama-3.2-1B and Llama-3-8B shaped workloads need
 * 5-50 MB; long many-token decode blocks and mixed batches without the
 * prefill kernel need more). Beside the prefill kernel, the launch of the
 * sequences with a few queries takes longer key pieces where that makes the
 * call fit (results as kv4_paged_attention's up to the float32 accumulation
 * order). All calls on one GPU share its array: two calls whose kernels may
 * run at the same time on one GPU (different streams, or the same stream
 * from several threads without ordering) race and give wrong results. The
 * array needs no initialization and keeps the last call's contents.
 */
#define KV4_NOALLOC_SCRATCH_BYTES (64u << 20)
kv4_status kv4_paged_attention_noalloc(const void* query, int64_t query_token_stride,
                                       const void* key_cache, const void* value_cache,
                                       const float* k_scale_cache, const float* v_scale_cache,
                                       int64_t num_blocks,
                                       const int32_t* block_table, int32_t max_blocks_per_seq,
                                       const int32_t* seq_lens, const int32_t* query_start_loc,
                                       int32_t num_seqs, int64_t num_q_tokens,
                                       int32_t max_query_len, int32_t max_seq_len,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_size, int32_t b, int32_t block_size,
                                       uint64_t sign_seed, float softmax_scale,
                                       void* out, void* stream);

/*
 * kv4_dequant -- gather and dequantize cache slots (for tests and debugging;
 * the round-trip check of [PR62881] Fix).
 *   out[t, h, i] = code * scale  (one float32 product), and with
 *   inverse_rotate != 0 additionally D.H(.)/b applied per head vector in
 *   float32, mapping back to the original domain.
 *   cache               uint8 [num_blocks, block_size, num_kv_heads, head_size/2]
 *   scale_cache         float32 [num_blocks, block_size, num_kv_heads]
 *   slot_mapping        int64 [num_tokens]; out-of-range slots give zeros
 *   out                 float32 [num_tokens, num_kv_heads, head_size]
 */
kv4_status kv4_dequant(const void* cache, const float* scale_cache, int64_t num_blocks,
                       const int64_t* slot_mapping, int64_t num_tokens,
                       int32_t num_kv_heads, int32_t head_size, int32_t b,
                       int32_t block_size, uint64_t sign_seed, int32_t inverse_rotate,
                       float* out, void* stream);

/*
 * Per-token-head INT8 / FP8 control modes: the pages' int8_per_token_head
 * and fp8_per_token_head ([PR56198]: controls that never use the transform;
 * [PR40835] review: int8 or FP8 cache dtype, the same float32 scale caches).
 * No rotation; one code byte per element. The rule is not on the pages and
 * is fixed here as symmetric absmax per (token, kv head) vector:
 *   KV4_MODE_INT8  scale = absmax / 127, code = clamp(rint_half_even(x /
 *                  scale), -128, 127) as a two's-complement byte;
 *   KV4_MODE_FP8   scale = absmax / 448, code = x / scale rounded to the
 *                  nearest OCP FP8 E4M3 (e4m3fn) value, ties to the even
 *                  mantissa, magnitudes >= 448 saturating to 448; the sign bit
 *                  follows the quotient's.
 * (IEEE float32 division; absmax == 0 stores scale 0 and code 0.) Caches:
 * uint8 [num_blocks, block_size, num_kv_heads, head_size], scales float32
 * [num_blocks, block_size, num_kv_heads].
 */
#define KV4_MODE_INT8 1
#define KV4_MODE_FP8 2

/*
 * kv4_pth_write -- write path of the int8 / fp8 modes: quantize each (token,
 * kv head) vector of key / value (bf16 [num_tokens, num_kv_heads, head_size],
 * token rows key_token_stride / value_token_stride elements apart) and store
 * it at slot_mapping[t] (slots outside [0, num_blocks * block_size) skip the
 * token). Arguments otherwise as kv4_rht_write; KV4_EINVAL for another mode.
 */
kv4_status kv4_pth_write(int32_t kv_quant_mode, const void* key, const void* value,
                         int64_t key_token_stride, int64_t value_token_stride,
                         void* key_cache, void* value_cache,
                         float* k_scale_cache, float* v_scale_cache,
                         const int64_t* slot_mapping, int64_t num_tokens,
                         int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                         int64_t num_blocks, void* stream);

/*
 * kv4_pth_attention_workspace_size / kv4_pth_attention -- the read path over
 * an int8 / fp8 per-token-head cache: as kv4_paged_attention_workspace_size /
 * kv4_paged_attention with no rotation, i.e. for each query head
 *   logit_j = k_scale_j * (q . value(code_K_j)) * softmax_scale,
 *   out = sum_j softmax(logit)_j * v_scale_j * value(code_V_j)  (bf16),
 * the same causal rule, GQA mapping, metadata, workspace contract, planner
 * overrides and error behaviour. Caches as written by kv4_pth_write with the
 * same kv_quant_mode; KV4_EINVAL for another mode.
 */
size_t kv4_pth_attention_workspace_size(int32_t kv_quant_mode, int64_t num_q_tokens,
                                        int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_size,
                                        int32_t max_query_len, int32_t max_seq_len);
kv4_status kv4_pth_attention(int32_t kv_quant_mode, const void* query, int64_t query_token_stride,
                             const void* key_cache, const void* value_cache,
                             const float* k_scale_cache, const float* v_scale_cache,
                             int64_t num_blocks,
                             const int32_t* block_table, int32_t max_blocks_per_seq,
                             const int32_t* seq_lens, const int32_t* query_start_loc,
                             int32_t num_seqs, int64_t num_q_tokens,
                             int32_t max_query_len, int32_t max_seq_len,
                             int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_size, int32_t block_size, float softmax_scale,
                             void* out, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * kv4_pth_dequant -- gather and dequantize int8 / fp8 cache slots (tests and
 * debugging): out[t, h, i] = value(code) * scale as one float32 product;
 * out-of-range slots give zeros. out float32 [num_tokens, num_kv_heads,
 * head_size].
 */
kv4_status kv4_pth_dequant(int32_t kv_quant_mode, const void* cache, const float* scale_cache,
                           int64_t num_blocks, const int64_t* slot_mapping, int64_t num_tokens,
                           int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                           float* out, void* stream);

/*
 * Cache layouts. Every entry point above takes the packed layout: codes
 * uint8 [num_blocks, block_size, num_kv_heads, C] (C = head_size / 2 for the
 * int4 RHT mode, head_size for int8 / fp8) and scales float32 [num_blocks,
 * block_size, num_kv_heads]. The *_layout entry points below take any
 * layout described by strides instead, for all three modes
 * (kv_quant_mode 0 = int4 RHT, KV4_MODE_INT8, KV4_MODE_FP8): the C code
 * bytes of (page p, token slot t of the page, kv head h) start at
 *   cache + p * block_stride + t * token_stride + h * head_stride
 * and its scale is the float at
 *   scale_cache + p * scale_block_stride + t * scale_token_stride
 *               + h * scale_head_stride
 * (the K and V caches share one layout). Code strides must be positive
 * multiples of 4 bytes (int4) or 8 bytes (int8 / fp8), scale strides
 * positive; the matrix-core kernels run where the code strides are also
 * multiples of 16 bytes, and serve one kv head per wave unless the heads of a
 * token slot are packed (head_stride == C, scale_head_stride == 1). Distinct
 * (page, slot, head) rows and scales must not overlap each other; the
 * library cannot check this, nor buffer sizes.
 */
typedef struct kv4_cache_layout {
  int64_t block_stride;        /* bytes between pages of a code cache          */
  int64_t token_stride;        /* bytes between token slots of a page          */
  int64_t head_stride;         /* bytes between kv heads of a token slot        */
  int64_t scale_block_stride;  /* floats between pages of a scale cache        */
  int64_t scale_token_stride;  /* floats between token slots                   */
  int64_t scale_head_stride;   /* floats between kv heads                      */
} kv4_cache_layout;

/* kv4_cache_layout_packed -- the packed layout of the other entry points. */
kv4_status kv4_cache_layout_packed(int32_t kv_quant_mode, int32_t num_kv_heads, int32_t head_size,
                                   int32_t block_size, kv4_cache_layout* layout);

/*
 * kv4_cache_layout_inline -- the inline-scale padded-slot layout of the
 * per-token-head caches (vLLM PR #40835 review of `_ensure_scale_caches`:
 * float32 views of sizes full_block = 2 kv_half_bytes, slot = num_kv_heads
 * padded rows, head = one padded row, scale offset = the code bytes of a row;
 * K scales in half 0 and V scales kv_half_bytes further; rows padded to a
 * 16-byte multiple, vLLM PR #62113 "16-byte-align per-token-head KV slots").
 * One buffer of num_blocks * block_bytes bytes holds both caches: page p is
 * the K half (block_size * num_kv_heads rows) then the V half; each row is C
 * code bytes, its float32 scale, then zero padding up to the pitch
 * P = round_up(C + 4, 16). Use key_cache = buffer, value_cache = buffer +
 * value_offset, k_scale_cache = (float*)(buffer + scale_offset),
 * v_scale_cache = (float*)(buffer + value_offset + scale_offset) with the
 * returned layout. block_bytes / value_offset / scale_offset may be NULL.
 */
kv4_status kv4_cache_layout_inline(int32_t kv_quant_mode, int32_t num_kv_heads, int32_t head_size,
                                   int32_t block_size, kv4_cache_layout* layout, int64_t* block_bytes,
                                   int64_t* value_offset, int64_t* scale_offset);

/*
 * kv4_write_layout / kv4_attention_layout_workspace_size /
 * kv4_attention_layout / kv4_dequant_layout -- kv4_rht_write,
 * kv4_paged_attention_workspace_size, kv4_paged_attention and kv4_dequant
 * (kv_quant_mode 0) or their kv4_pth_* counterparts (modes 1 / 2: b,
 * sign_seed and inverse_rotate are ignored) over caches in `layout`. Same
 * results, argument rules and errors, plus KV4_EINVAL for an invalid layout.
 * The workspace size depends on the layout (it selects the plan).
 *
 * kv4_attention_layout also takes sliding_window (0 = off): the query at
 * position p then sees only keys j with p - sliding_window < j <= p, the
 * window most recent keys of its causal range (the pages' "added window"
 * commit of vLLM PR #40835 names the feature; this rule is the reading taken
 * here). Keys below every row's window are not read. Negative values give
 * KV4_EINVAL. Pass the packed layout (kv4_cache_layout_packed) for the caches
 * of the other entry points.
 */
kv4_status kv4_write_layout(int32_t kv_quant_mode, const void* key, const void* value,
                            int64_t key_token_stride, int64_t value_token_stride,
                            void* key_cache, void* value_cache,
                            float* k_scale_cache, float* v_scale_cache,
                            const kv4_cache_layout* layout,
                            const int64_t* slot_mapping, int64_t num_tokens,
                            int32_t num_kv_heads, int32_t head_size, int32_t b,
                            int32_t block_size, int64_t num_blocks,
                            uint64_t sign_seed, void* stream);
size_t kv4_attention_layout_workspace_size(int32_t kv_quant_mode, const kv4_cache_layout* layout,
                                           int64_t num_q_tokens, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_size, int32_t max_query_len,
                                           int32_t max_seq_len);
kv4_status kv4_attention_layout(int32_t kv_quant_mode, const void* query, int64_t query_token_stride,
                                const void* key_cache, const void* value_cache,
                                const float* k_scale_cache, const float* v_scale_cache,
                                const kv4_cache_layout* layout, int64_t num_blocks,
                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, const int32_t* query_start_loc,
                                int32_t num_seqs, int64_t num_q_tokens,
                                int32_t max_query_len, int32_t max_seq_len,
                                int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_size, int32_t b, int32_t block_size,
                                uint64_t sign_seed, int32_t sliding_window, float softmax_scale,
                                void* out, void* workspace, size_t workspace_bytes,
                                void* stream);
kv4_status kv4_dequant_layout(int32_t kv_quant_mode, const void* cache, const float* scale_cache,
                              const kv4_cache_layout* layout, int64_t num_blocks,
                              const int64_t* slot_mapping, int64_t num_tokens,
                              int32_t num_kv_heads, int32_t head_size, int32_t b,
                              int32_t block_size, uint64_t sign_seed, int32_t inverse_rotate,
                              float* out, void* stream);

/*
 * kv4_stream_read -- measurement aid, not a step of the method: reads `bytes`
 * (a multiple of 16) of device memory at `buffer` (16-byte aligned) once,
 * with 16-byte non-temporal vector loads from `grid` workgroups of 256
 * lanes, four loads in flight per lane. Its duration gives the achievable
 * HBM read rate that the attention kernels' bandwidth is compared with.
 * `sink` (4 bytes, device) receives a value only if the XOR of everything
 * read is 0x9E3779B9 (which keeps the loads from being optimized away).
 */
kv4_status kv4_stream_read(const void* buffer, int64_t bytes, uint32_t* sink, int32_t grid,
                           void* stream);

/*
 * kv4_debug_flags -- the inputs the kernels of the current device clamped or
 * skipped since the last clear, as KV4_DEBUG_* bits (libraries built with
 * -DKV4_DEBUG; build.build_debug_library()). Every kernel keeps its
 * accesses inside the caller's buffers whatever the metadata holds: a
 * negative slot is padding (skipped, by contract); a slot past the cache, a
 * page id outside [0, num_blocks), a seq_len beyond the page table or a
 * query_start_loc entry outside [0, num_q_tokens] or decreasing is treated
 * as "no data" or clamped. Debug builds also record each such event (one
 * bit per kind, any kernel of the library) instead of only absorbing it.
 * Synchronizes the current device first, so earlier calls on every stream
 * are counted; with `clear` nonzero the flags are reset after the read.
 * `flags` is a host pointer. Release builds: KV4_EUNSUPPORTED, *flags = 0.
 */
#define KV4_DEBUG_SLOT 1u     /* a write or dequant slot >= num_blocks * block_size */
#define KV4_DEBUG_PAGE 2u     /* a block_table entry outside [0, num_blocks) */
#define KV4_DEBUG_SEQLEN 4u   /* a seq_len < 0 or beyond max_blocks_per_seq * block_size */
#define KV4_DEBUG_QSL 8u      /* a query_start_loc entry outside [0, num_q_tokens], or decreasing */
kv4_status kv4_debug_flags(uint32_t* flags, int32_t clear);

/*
 * kv4_last_error -- thread-local description of the last failure of a call
 * made on this thread ("" after a call that succeeded). Never NULL; the
 * string stays valid until the next kv4_* call on the same thread.
 */
const char* kv4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KV4_H_ */
