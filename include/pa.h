/*
 * pa.h - C ABI of the MI355X (gfx950) paged-KV-cache attention library.
 *
 * The library computes scaled-dot-product attention softmax(Q K^T * scale) V
 * for continuous batching: new query tokens of many sequences arrive packed
 * back to back, each sequence keeps its keys/values in a paged KV cache that
 * is addressed through a per-sequence block table, query head h reads KV head
 * floor(h / (num_heads / num_kv_heads)) (grouped-query attention), and new
 * query row i of sequence b sees KV positions 0 .. past_b + i, where
 * past_b = seqlens_kv[b] - q_len_b.
 *
 * Sources: onnxruntime pull request #31611, "[WebGPU] Initial PagedAttention
 * implementation (1/n)" - sections "Description" (scatter of new K/V into the
 * paged cache, packed varlen queries, packed (token_count, hidden_size)
 * output) and "FlashAttention: optional seqlens_q input" (per-sequence past
 * length = total KV length minus that sequence's own query length), and the
 * maintainer review's list of checked items (token-to-sequence scan, causal
 * length past + q + 1, scatter block addressing, GQA mapping); onnx-light
 * operator page "FlexAttention" - sections "FlexAttention Computation" and
 * "Grouped Query Attention (GQA)".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is DEVICE memory owned by the caller, except the
 *   output arguments of pa_profile_read / pa_validate_metadata, which are
 *   host memory.  The library allocates no device memory and keeps no
 *   pointer after a call returns.
 * - `stream` is a hipStream_t passed as void*; NULL is the null stream.  All
 *   kernels are enqueued on it; pa_scatter_kv and pa_attention never
 *   synchronise the host (no device-to-host copies).  Apart from kernel
 *   launches they enqueue nothing (no memset or copy), so a stream capture
 *   can record them into a graph that is replayed later.
 * - Element type `dtype`: PA_F16 (IEEE binary16) or PA_BF16 (bfloat16) for
 *   Q, new K/V, the caches and the output.  Arithmetic is fp32: QK^T and
 *   P.V accumulate in fp32 (matrix cores), the softmax runs in fp32, P is
 *   rounded to dtype for the P.V product, and the output is rounded to
 *   dtype with round-to-nearest-even.
 * - Cache layout (both caches): [num_blocks, block_size, num_kv_heads,
 *   head_size], row-major; cache slot s = block * block_size + offset holds
 *   one token's num_kv_heads * head_size row.
 * - Index arrays are int32.  Offsets into q, out, the caches and the
 *   workspace are computed in 64 bits; offsets inside one cache block and
 *   the work-item counts are 32-bit, which the size limits of each entry
 *   point keep in range.
 * - Errors: argument checks happen on the host before any HIP call and
 *   return PA_ERR_INVALID_ARGUMENT / PA_ERR_NOT_IMPLEMENTED /
 *   PA_ERR_WORKSPACE_TOO_SMALL; a failed kernel launch returns PA_ERR_HIP.
 *   pa_last_error() gives a message for the calling thread's last failure.
 *   Device-resident metadata (cu_seqlens_q, seqlens_kv, block_table,
 *   slot_mapping) are trusted preconditions; pa_validate_metadata checks
 *   them (debug/test use only).  No C++ exception crosses this ABI.
 * - Calls are stateless and re-entrant: concurrent calls on different
 *   streams with different workspaces do not interfere.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Status codes.
 *
 * Defines: the error convention of "[WebGPU] Initial PagedAttention
 * implementation (1/n)":
 * - section "Description": the v1 op rejects the options it does not
 *   support (softcap, local_window_size, bfloat16) up front with
 *   NOT_IMPLEMENTED; the maintainer review's second cross-cutting point and
 *   the author's reply do the same for the KV-cache quantization option.
 *   Here: a shape or option outside this library's limits (head size,
 *   block size, group size, context length, dtype) is
 *   PA_ERR_NOT_IMPLEMENTED, returned before any HIP call.
 * - the design document quoted in the page's later review rounds
 *   ("Cache-output aliasing"): a violated argument contract (there, cache
 *   outputs that do not alias the inputs) fails with INVALID_ARGUMENT, as
 *   the CUDA op does.  Here: a null pointer, a misaligned buffer, a count
 *   out of range or a non-finite scale is PA_ERR_INVALID_ARGUMENT.
 * PA_ERR_WORKSPACE_TOO_SMALL (a workspace below the size this library
 * reports) and PA_ERR_HIP (a failed kernel launch) are this library's own.
 */
typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = 1,
  PA_ERR_NOT_IMPLEMENTED = 2,
  PA_ERR_WORKSPACE_TOO_SMALL = 3,
  PA_ERR_HIP = 4
} pa_status_t;

typedef enum pa_dtype { PA_F16 = 0, PA_BF16 = 1 } pa_dtype_t;

/*
 * pa_scatter_kv - write this step's new K/V rows into the paged caches.
 *
 * Defines: the scatter step of "[WebGPU] Initial PagedAttention
 * implementation (1/n)", section "Description" (new keys/values go into
 * their block slots before attention reads the cache).
 *
 *   for t in [0, num_tokens): s = slot_mapping[t]; if s >= 0:
 *       k_cache[s / block_size][s % block_size][:][:] = k_new[t][:][:]
 *       v_cache[s / block_size][s % block_size][:][:] = v_new[t][:][:]
 *
 * k_new, v_new   [num_tokens, num_kv_heads, head_size] dtype, read only.
 * slot_mapping   [num_tokens] int32; a negative slot skips the token.
 *                Non-negative slots must be unique and < num_blocks *
 *                block_size (precondition; duplicates race).
 * k_cache,
 * v_cache        [num_blocks, block_size, num_kv_heads, head_size] dtype,
 *                updated in place.  Bytes are copied verbatim (bit-exact).
 * Limits: head_size % 8 == 0, num_kv_heads >= 1, block_size >= 1,
 * num_blocks * block_size <= INT32_MAX.  k_new, v_new and the caches must be
 * 16-byte aligned (else PA_ERR_INVALID_ARGUMENT).  num_tokens == 0 returns
 * PA_OK without launching.
 */
pa_status_t pa_scatter_kv(const void* k_new, const void* v_new,
                          const int32_t* slot_mapping, void* k_cache,
                          void* v_cache, int64_t num_tokens,
                          int64_t num_blocks, int32_t num_kv_heads,
                          int32_t head_size, int32_t block_size,
                          int32_t dtype, void* stream);

/*
 * pa_scatter_kv_paged - pa_scatter_kv with each new token's slot computed on
 * the device from the batch metadata instead of a slot_mapping array.
 *
 * Defines: "[WebGPU] Initial PagedAttention implementation (1/n)", section
 * "Description" (the op derives the cache slots of the new tokens from the
 * cumulative query lengths, the past lengths and the block table) and the
 * review's checked items (token-to-sequence scan, scatter block
 * addressing).  For new token t: b = the first sequence with
 * cu_seqlens_q[b+1] > t; past_b = seqlens_kv[b] - q_len_b;
 * pos = past_b + (t - cu_seqlens_q[b]);
 *   s = block_table[b][pos / block_size] * block_size + pos % block_size,
 * then the copy of pa_scatter_kv.  A negative table entry skips the token.
 *
 * k_new, v_new   [num_tokens, num_kv_heads, head_size] dtype, read only.
 * cu_seqlens_q, seqlens_kv, block_table
 *                as for pa_attention (same preconditions: past_b >= 0 and
 *                pos / block_size < max_blocks_per_seq for every token).
 * k_cache,
 * v_cache        [num_blocks, block_size, num_kv_heads, head_size], updated
 *                in place, bit-exact copies.  The slots must not repeat
 *                (precondition; they do not when the table rows are
 *                disjoint, as a block manager hands them out).
 * Limits: as pa_scatter_kv, plus num_seqs >= 1, max_blocks_per_seq >= 1,
 * max_blocks_per_seq * block_size <= INT32_MAX.  num_tokens == 0 returns
 * PA_OK without launching.
 */
pa_status_t pa_scatter_kv_paged(const void* k_new, const void* v_new,
                                const int32_t* cu_seqlens_q,
                                const int32_t* seqlens_kv,
                                const int32_t* block_table, void* k_cache,
                                void* v_cache, int32_t num_seqs,
                                int64_t num_tokens, int32_t max_blocks_per_seq,
                                int64_t num_blocks, int32_t num_kv_heads,
                                int32_t head_size, int32_t block_size,
                                int32_t dtype, void* stream);

/*
 * pa_seqlens_from_past - total KV lengths from past lengths, on the device:
 *   seqlens_kv[b] = past_seqlens[b] + (cu_seqlens_q[b+1] - cu_seqlens_q[b]).
 *
 * Defines: "[WebGPU] Initial PagedAttention implementation (1/n)", section
 * "FlashAttention: optional seqlens_q input" (the op receives past lengths;
 * past_b = total_b - q_len_b).  Lets a caller that holds past lengths feed
 * pa_scatter_kv_paged and pa_attention, which take total lengths.
 * cu_seqlens_q [num_seqs + 1], past_seqlens [num_seqs] int32, read only;
 * seqlens_kv [num_seqs] int32, written (may not alias the inputs).
 * num_seqs >= 1.
 */
pa_status_t pa_seqlens_from_past(const int32_t* cu_seqlens_q,
                                 const int32_t* past_seqlens,
                                 int32_t* seqlens_kv, int32_t num_seqs,
                                 void* stream);

/*
 * pa_rotary_scatter_kv - the steps ahead of the attention for one batch of
 * new tokens, fused: split packed QKV rows, rotate Q and K by the rotary
 * position embedding at each token's KV position, write the rotated Q to
 * q_out and the rotated K and plain V into the paged caches at the slots
 * the block table gives (as pa_scatter_kv_paged).
 *
 * Defines: "[WebGPU] Initial PagedAttention implementation (1/n)": the file
 * summaries (a packed-QKV split program and a rotary program run ahead of
 * the scatter) and the review's summary (interleaved and split pairing,
 * the rotation's sign, pass-through of dimensions >= rotary_dim).  The
 * pages define no formula; this library's reading is the rotary position
 * embedding of Su et al. (RoFormer): for token i of sequence b at position
 * p = past_b + i and pair k < rotary_dim / 2 with dimensions (x_a, x_b) =
 * (2k, 2k+1) when interleaved, (k, k + rotary_dim / 2) otherwise:
 *   x_a' = x_a cos - x_b sin,  x_b' = x_b cos + x_a sin,
 *   cos = cos_cache[p][k], sin = sin_cache[p][k];
 * dimensions >= rotary_dim are copied.  Computed in fp32 from the dtype
 * inputs, rounded once to dtype (nearest even).
 *
 * query        [num_tokens, num_heads, head_size] dtype, or, when key and
 *              value are NULL, packed rows [num_tokens, num_heads +
 *              2 num_kv_heads, head_size]: each token's Q heads, then its K
 *              heads, then its V heads.  NULL with key, value given and
 *              q_out NULL (a K/V-only rotated scatter, such as filling the
 *              cache with history keys).
 * key, value   [num_tokens, num_kv_heads, head_size] dtype, or both NULL.
 * cos_cache,
 * sin_cache    [max_position, rotary_dim / 2] dtype, or both NULL (no
 *              rotation: a split and scatter only).
 * rotary_dim   multiple of 16 in [16, head_size] (others:
 *              NOT_IMPLEMENTED); ignored without tables.
 * interleaved  nonzero: interleaved pairing; 0: split pairing.
 * cu_seqlens_q, seqlens_kv, block_table
 *              as for pa_attention.  A negative table entry gives the token
 *              no cache slot (its K/V are not written; its Q is).
 * q_out        [num_tokens, num_heads, head_size] dtype, written (the Q
 *              pa_attention then reads); must not overlap the inputs.  NULL:
 *              the Q rows are not written (pa_attention_rope then reads Q
 *              from the packed rows and rotates it as it loads it).
 * k_cache,
 * v_cache      paged caches, updated in place.
 * All tensor pointers 16-byte aligned (else PA_ERR_INVALID_ARGUMENT).
 * A token whose position is >= max_position (with tables) or negative
 * (seqlens_kv[b] < q_len_b) breaks a precondition and is skipped whole:
 * its q_out rows and cache slot are left as they were.
 * Limits: head_size a multiple of 8; num_blocks * block_size and
 * max_blocks_per_seq * block_size <= INT32_MAX.  num_tokens == 0 returns
 * PA_OK without launching.
 */
pa_status_t pa_rotary_scatter_kv(const void* query, const void* key,
                                 const void* value, const void* cos_cache,
                                 const void* sin_cache, int32_t max_position,
                                 int32_t rotary_dim, int32_t interleaved,
                                 const int32_t* cu_seqlens_q,
                                 const int32_t* seqlens_kv,
                                 const int32_t* block_table, void* q_out,
                                 void* k_cache, void* v_cache, int32_t num_seqs,
                                 int64_t num_tokens, int32_t max_blocks_per_seq,
                                 int64_t num_blocks, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_size,
                                 int32_t block_size, int32_t dtype, void* stream);


/*
 * pa_rotary_scatter_kv_fp8 - pa_rotary_scatter_kv into fp8 (e4m3) caches
 * with per-channel scales (pa_scatter_kv_fp8's format).
 *
 * Defines: the rotary step of pa_rotary_scatter_kv (same pages and
 * sections) ahead of the quantized KV cache of "[WebGPU] Initial
 * PagedAttention implementation (1/n)", "Roadmap", phase 3.  Each K row is
 * rotated and rounded to dtype exactly as pa_rotary_scatter_kv does, then it
 * and each V row are quantized as pa_scatter_kv_fp8 quantizes: the cache
 * codes are bitwise those of pa_rotary_scatter_kv into 16-bit caches
 * followed by pa_scatter_kv_fp8 of the rotated rows.  Q (q_out) is written
 * in dtype as by pa_rotary_scatter_kv, or skipped when q_out is NULL.
 *
 * k_scale,
 * v_scale      [num_kv_heads, head_size] float32, 16-byte aligned.
 * k_cache,
 * v_cache      [num_blocks, block_size, num_kv_heads, head_size] uint8 e4m3
 *              codes, updated in place.
 * Every other argument, limit and status code as for pa_rotary_scatter_kv;
 * a null scale pointer returns PA_ERR_INVALID_ARGUMENT.
 */
pa_status_t pa_rotary_scatter_kv_fp8(const void* query, const void* key,
                                     const void* value, const void* cos_cache,
                                     const void* sin_cache, int32_t max_position,
                                     int32_t rotary_dim, int32_t interleaved,
                                     const int32_t* cu_seqlens_q,
                                     const int32_t* seqlens_kv,
                                     const int32_t* block_table,
                                     const float* k_scale, const float* v_scale,
                                     void* q_out, void* k_cache, void* v_cache,
                                     int32_t num_seqs, int64_t num_tokens,
                                     int32_t max_blocks_per_seq,
                                     int64_t num_blocks, int32_t num_heads,
                                     int32_t num_kv_heads, int32_t head_size,
                                     int32_t block_size, int32_t dtype,
                                     void* stream);

/*
 * pa_attention_workspace_size - bytes of device workspace pa_attention
 * needs for these host-known sizes (an upper bound over every metadata the
 * device could hold).  Returns 0 when the sizes are invalid.
 *
 * Defines: the scratch-buffer sizing of "[WebGPU] Initial PagedAttention
 * implementation (1/n)": the review names WebGPU resource limits (checked
 * dispatch size, scratch-buffer and storage-binding limits) as a finding
 * area and the author's reply takes them on; "Roadmap" defers graph capture
 * until an attention-metadata sizing bound exists.  This library's reading:
 * every grid and scratch size comes from host-known bounds alone (counts
 * and max_blocks_per_seq, never device metadata), so the size is known
 * before the call, needs no readback, and suits capture.
 */
size_t pa_attention_workspace_size(int32_t num_seqs, int64_t num_tokens,
                                   int32_t max_blocks_per_seq,
                                   int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size);

/*
 * pa_attention - paged causal GQA attention over packed varlen queries.
 *
 * Defines: "[WebGPU] Initial PagedAttention implementation (1/n)", sections
 * "Description" and "FlashAttention: optional seqlens_q input"; the math is
 * the "FlexAttention Computation" of the FlexAttention operator page with
 * its GQA head mapping and masked scores treated as -inf.
 *
 * For sequence b: q_len_b = cu_seqlens_q[b+1] - cu_seqlens_q[b],
 * L_b = seqlens_kv[b], past_b = L_b - q_len_b; for new row i < q_len_b
 * (packed token t = cu_seqlens_q[b] + i) and query head h:
 *   K_j = k_cache[block_table[b][j / block_size]][j % block_size][h / G]
 *   out[t][h] = sum_{j <= past_b + i} softmax_j(scale * q[t][h] . K_j) V_j
 * with G = num_heads / num_kv_heads.
 *
 * q            [num_tokens, num_heads, head_size] dtype (packed tokens).
 * cu_seqlens_q [num_seqs + 1] int32: cu[0] = 0, nondecreasing,
 *              cu[num_seqs] = num_tokens.  Empty sequences are allowed.
 * seqlens_kv   [num_seqs] int32: total KV length of each sequence including
 *              this step's tokens; must be >= q_len_b (precondition) and
 *              <= max_blocks_per_seq * block_size.
 * block_table  [num_seqs, max_blocks_per_seq] int32 row-major; entries
 *              0 .. ceil(L_b / block_size) - 1 of row b must be valid block
 *              ids (< num_blocks); later entries are never read.  Blocks may
 *              be shared between sequences.
 * k_cache,
 * v_cache      paged caches as above; read only.  Slots beyond L_b and
 *              blocks not referenced are never read into the result (they
 *              may hold NaN).
 * out          [num_tokens, num_heads, head_size] dtype, fully written.
 * scale        finite float, used exactly as given (0 gives the mean of the
 *              visible V rows).
 * softcap      score soft cap c: finite, >= 0.  c > 0 replaces every scaled
 *              score x = scale * q . K_j by c * tanh(x / c) before the mask
 *              and the softmax; 0 turns it off.  The PagedAttention page
 *              names the option ("Description"; "Roadmap", phase 2 lifts
 *              it) without defining it: this is the library's reading.
 *              PA_ERR_INVALID_ARGUMENT for a negative or non-finite c, or
 *              when scale / c overflows float.
 * local_window_size
 *              sliding window W: W > 0 limits new row i to its last W keys,
 *              past_b + i - W < j <= past_b + i (same page and sections,
 *              same reading); W <= 0 turns it off.  Whole 1024-key splits
 *              (rows of sequences with q_len_b * G <= 16) and 64-key tiles
 *              (other rows) before the window of a sequence's first new
 *              row are skipped: those cache slots are not read.
 * workspace    device buffer of at least pa_attention_workspace_size(...)
 *              bytes, 256-byte aligned; contents need no initialisation and
 *              are scratch (plan lists, split-KV partial results).
 * Limits: head_size in {64, 128}; block_size a power of two in [16, 1024];
 * num_heads % num_kv_heads == 0 with G <= 128; num_blocks * block_size
 * <= INT32_MAX; max_blocks_per_seq * block_size <= 262144 tokens;
 * num_seqs <= 65536; block_size * num_kv_heads * head_size * 2 (the bytes
 * of one cache block) <= INT32_MAX; and the work the sizes can produce fits
 * the kernels' 32-bit counts: num_seqs * ceil(max_blocks_per_seq *
 * block_size / 1024) * num_kv_heads decode items, the prefill tile items
 * and the split-KV partial rows each <= 2^30.  Other shapes return
 * PA_ERR_NOT_IMPLEMENTED (pa_attention_workspace_size returns 0 for them).
 * q, out and the caches must be 16-byte aligned (else
 * PA_ERR_INVALID_ARGUMENT), and out must not overlap q (else
 * PA_ERR_INVALID_ARGUMENT: other work-groups still read q while out is
 * written).  num_tokens == 0 returns PA_OK without launching.
 */
pa_status_t pa_attention(const void* q, const int32_t* cu_seqlens_q,
                         const int32_t* seqlens_kv, const int32_t* block_table,
                         const void* k_cache, const void* v_cache, void* out,
                         int32_t num_seqs, int64_t num_tokens,
                         int32_t max_blocks_per_seq, int64_t num_blocks,
                         float scale, float softcap, int32_t local_window_size,
                         int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_size, int32_t block_size, int32_t dtype,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * pa_attention_rope - pa_attention with the rotary embedding of Q fused into
 * the attention's Q load, reading Q from rows of any stride (such as the
 * packed QKV rows that pa_rotary_scatter_kv splits).
 *
 * Defines: "[WebGPU] Initial PagedAttention implementation (1/n)": the file
 * summaries put a packed-QKV split program and a rotary program ahead of the
 * attention, each a round trip through memory.  Here pa_rotary_scatter_kv
 * (q_out NULL) rotates and scatters K and V, and this call reads the
 * unrotated Q straight from the packed rows and rotates it on load, so Q is
 * neither written nor read back.  The rotation is pa_rotary_scatter_kv's
 * (same pairing, position p = past_b + i, tables, fp32 arithmetic rounded
 * once to dtype): the result is bitwise that of pa_rotary_scatter_kv with a
 * q_out followed by pa_attention on q_out.
 *
 * q            element (t, h, d) of Q at q[t * q_row_stride + h * head_size
 *              + d], dtype; for packed [num_tokens, num_heads + 2
 *              num_kv_heads, head_size] rows, q is the packed buffer and
 *              q_row_stride = (num_heads + 2 num_kv_heads) * head_size.
 * q_row_stride >= num_heads * head_size, a multiple of 8 (16-byte rows), and
 *              num_tokens * q_row_stride <= 2^60; else
 *              PA_ERR_INVALID_ARGUMENT.
 * cos_cache,
 * sin_cache    [max_position, rotary_dim / 2] dtype, 16-byte aligned, or
 *              both NULL (no rotation: pa_attention on strided Q rows).
 * rotary_dim   multiple of 16 in [16, head_size] (others: NOT_IMPLEMENTED;
 *              outside [1, head_size]: INVALID_ARGUMENT); dimensions >=
 *              rotary_dim are used as given.  Ignored without tables.
 * interleaved  nonzero: pairs (2k, 2k+1); 0: pairs (k, k + rotary_dim / 2).
 * max_position >= 1 with tables.  A row whose position is >= max_position
 *              breaks a precondition and is used unrotated.
 * Every other argument, limit, status code and the empty call as for
 * pa_attention; out must not overlap q's rows (else INVALID_ARGUMENT).
 */
pa_status_t pa_attention_rope(const void* q, int64_t q_row_stride,
                              const void* cos_cache, const void* sin_cache,
                              int32_t max_position, int32_t rotary_dim,
                              int32_t interleaved, const int32_t* cu_seqlens_q,
                              const int32_t* seqlens_kv,
                              const int32_t* block_table, const void* k_cache,
                              const void* v_cache, void* out, int32_t num_seqs,
                              int64_t num_tokens, int32_t max_blocks_per_seq,
                              int64_t num_blocks, float scale, float softcap,
                              int32_t local_window_size, int32_t num_heads,
                              int32_t num_kv_heads, int32_t head_size,
                              int32_t block_size, int32_t dtype, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * pa_attention_noalloc - pa_attention without a caller workspace and
 * without any device allocation in the call.
 *
 * For callers that cannot allocate device memory around the call: code
 * under stream/graph capture, tight serving loops, harnesses that forbid
 * allocation.  The result is pa_attention's, from the same kernels; the plan
 * lists, fetch counters and split-KV partials live in a fixed 256 MiB
 * device-resident scratch array inside the library (one per GPU, held until
 * the process ends, set up on the first call on each device).
 *
 * Arguments, limits, status codes and empty calls as for pa_attention,
 * minus workspace / workspace_bytes.  Sizes whose workspace
 * (pa_attention_workspace_size) exceeds 256 MiB return
 * PA_ERR_WORKSPACE_TOO_SMALL before any HIP call (the decode- and
 * prefill-shaped batches this library is measured on need 33 MiB and
 * 3 MiB; a mixed batch of 256 sequences with 32768-token tables needs more:
 * use pa_attention there).  The call launches kernels only (no allocation,
 * memset or copy); the plan kernel initialises what must start at zero.
 *
 * All calls on one GPU share that GPU's scratch, which keeps the last
 * call's contents: calls that overlap in time on one GPU (concurrent
 * streams, or threads) race and must be serialised by the caller.
 */
pa_status_t pa_attention_noalloc(const void* q, const int32_t* cu_seqlens_q,
                                 const int32_t* seqlens_kv,
                                 const int32_t* block_table,
                                 const void* k_cache, const void* v_cache,
                                 void* out, int32_t num_seqs, int64_t num_tokens,
                                 int32_t max_blocks_per_seq, int64_t num_blocks,
                                 float scale, float softcap,
                                 int32_t local_window_size, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_size,
                                 int32_t block_size, int32_t dtype, void* stream);

/*
 * pa_scatter_kv_fp8 - pa_scatter_kv into fp8 caches: each new K/V element is
 * quantized to an 8-bit float with a per-(KV head, channel) scale.
 *
 * Defines: the quantized KV cache of "[WebGPU] Initial PagedAttention
 * implementation (1/n)", section "Roadmap" (phase 3: a cache element type
 * apart from the query type, quantized KV first).  The page fixes no
 * format; this library's reading: cache elements are OCP e4m3 (4 exponent
 * bits, bias 7, 3 mantissa bits, largest finite 448, no infinities) and
 *   code(x) = e4m3_round(sat(fp32(x) * fp32(1 / scale[h][d])))
 * with 1/scale and the product rounded to float32, sat() clamping
 * magnitudes above 448 (infinities included) to 448, and e4m3_round()
 * rounding to the nearest e4m3 value, ties to the even mantissa (a NaN
 * input gives a NaN code).  Element value on read: e4m3(code) * scale.
 *
 * k_new, v_new   [num_tokens, num_kv_heads, head_size] dtype, read only.
 * slot_mapping   [num_tokens] int32, as for pa_scatter_kv.
 * k_scale,
 * v_scale        [num_kv_heads, head_size] float32, read only; finite and
 *                > 0 (precondition).
 * k_cache,
 * v_cache        [num_blocks, block_size, num_kv_heads, head_size] uint8
 *                e4m3 codes, updated in place.
 * Limits and empty calls as for pa_scatter_kv.  Bit-exact with the
 * definition above.
 */
pa_status_t pa_scatter_kv_fp8(const void* k_new, const void* v_new,
                              const int32_t* slot_mapping, const float* k_scale,
                              const float* v_scale, void* k_cache, void* v_cache,
                              int64_t num_tokens, int64_t num_blocks,
                              int32_t num_kv_heads, int32_t head_size,
                              int32_t block_size, int32_t dtype, void* stream);

/*
 * pa_scatter_kv_paged_fp8 - pa_scatter_kv_fp8 with each new token's slot
 * computed on the device from the batch metadata, as pa_scatter_kv_paged
 * computes it.
 *
 * Defines: the slot derivation of "[WebGPU] Initial PagedAttention
 * implementation (1/n)", section "Description" (slots from the cumulative
 * query lengths, the past lengths and the block table), into the quantized
 * cache of section "Roadmap" (phase 3).  For new token t the slot s is
 * pa_scatter_kv_paged's; the codes written at s are pa_scatter_kv_fp8's
 * (same quantization, same per-channel scales).  A negative table entry
 * skips the token.
 *
 * k_new, v_new, cu_seqlens_q, seqlens_kv, block_table
 *                as for pa_scatter_kv_paged.
 * k_scale,
 * v_scale        as for pa_scatter_kv_fp8 (16-byte aligned).
 * k_cache,
 * v_cache        [num_blocks, block_size, num_kv_heads, head_size] uint8
 *                e4m3 codes, updated in place.
 * Limits, status codes and empty calls as for pa_scatter_kv_paged; null or
 * misaligned scales are PA_ERR_INVALID_ARGUMENT.  Bit-exact: the caches
 * equal pa_scatter_kv_fp8's with the slots pa_scatter_kv_paged derives.
 */
pa_status_t pa_scatter_kv_paged_fp8(const void* k_new, const void* v_new,
                                    const int32_t* cu_seqlens_q,
                                    const int32_t* seqlens_kv,
                                    const int32_t* block_table,
                                    const float* k_scale, const float* v_scale,
                                    void* k_cache, void* v_cache,
                                    int32_t num_seqs, int64_t num_tokens,
                                    int32_t max_blocks_per_seq,
                                    int64_t num_blocks, int32_t num_kv_heads,
                                    int32_t head_size, int32_t block_size,
                                    int32_t dtype, void* stream);

/*
 * pa_attention_fp8 - pa_attention over fp8 caches written by
 * pa_scatter_kv_fp8, for decode-shaped batches.
 *
 * Defines: pa_attention's result with K_j and V_j replaced by their
 * dequantized values e4m3(code) * scale[h / G][d] (section "Roadmap" of
 * the PagedAttention page, phase 3, quantized KV in the decode path).
 *
 * Arguments (softcap and local_window_size included) as for pa_attention,
 * plus:
 * k_cache,
 * v_cache      [num_blocks, block_size, num_kv_heads, head_size] uint8
 *              e4m3 codes; read only.
 * k_scale,
 * v_scale      [num_kv_heads, head_size] float32, read only.
 * max_q_len    host-known upper bound of every q_len_b; max_q_len * G must
 *              be <= 16 (one decode tile of query columns: decode steps and
 *              short speculative chunks), else PA_ERR_NOT_IMPLEMENTED.  A
 *              sequence whose q_len_b * G exceeds 16 despite the bound
 *              (precondition violation) gets no work: its output rows are
 *              left unwritten.
 * workspace    at least pa_attention_workspace_size(...) bytes, as for
 *              pa_attention.
 * Other limits, status codes and empty calls as for pa_attention.
 */
pa_status_t pa_attention_fp8(const void* q, const int32_t* cu_seqlens_q,
                             const int32_t* seqlens_kv, const int32_t* block_table,
                             const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale, void* out,
                             int32_t num_seqs, int64_t num_tokens, int32_t max_q_len,
                             int32_t max_blocks_per_seq, int64_t num_blocks,
                             float scale, float softcap, int32_t local_window_size,
                             int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_size, int32_t block_size, int32_t dtype,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_attention_rope_fp8 - pa_attention_fp8 with Q read from strided (for
 * example packed QKV) rows and rotated as it is loaded, as
 * pa_attention_rope does over 16-bit caches.
 *
 * Defines: the rotary program that runs just ahead of the attention in
 * "[WebGPU] Initial PagedAttention implementation (1/n)" (the file
 * summaries: a packed-QKV split and a rotary program ahead of the scatter;
 * the review's summary: interleaved or split pairing, pass-through of
 * dimensions >= rotary_dim), fused into the Q load of the quantized-cache
 * attention of section "Roadmap" (phase 3).  The rotation is
 * pa_attention_rope's (position p = past_b + i, fp32 arithmetic rounded
 * once to dtype), applied before the K scale is folded into Q, so the
 * result is bitwise that of pa_rotary_scatter_kv_fp8 with a q_out followed
 * by pa_attention_fp8 on q_out.
 *
 * q, q_row_stride, cos_cache, sin_cache, rotary_dim, interleaved,
 * max_position   as for pa_attention_rope.
 * Every other argument (k_scale, v_scale, max_q_len included), limit,
 * status code and the empty call as for pa_attention_fp8; out must not
 * overlap q's rows (else PA_ERR_INVALID_ARGUMENT).
 */
pa_status_t pa_attention_rope_fp8(const void* q, int64_t q_row_stride,
                                  const void* cos_cache, const void* sin_cache,
                                  int32_t max_position, int32_t rotary_dim,
                                  int32_t interleaved,
                                  const int32_t* cu_seqlens_q,
                                  const int32_t* seqlens_kv,
                                  const int32_t* block_table,
                                  const void* k_cache, const void* v_cache,
                                  const float* k_scale, const float* v_scale,
                                  void* out, int32_t num_seqs,
                                  int64_t num_tokens, int32_t max_q_len,
                                  int32_t max_blocks_per_seq,
                                  int64_t num_blocks, float scale,
                                  float softcap, int32_t local_window_size,
                                  int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_size, int32_t block_size,
                                  int32_t dtype, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * pa_validate_metadata - debug/test check of the device metadata that
 * pa_attention / pa_scatter_kv trust.
 *
 * Defines: the maintainer review of "[WebGPU] Initial PagedAttention
 * implementation (1/n)" ("Summary": findings concentrated on host-side
 * validation of device-derived values; first cross-cutting point: two
 * blocking device-to-host readbacks of the metadata per node and run, which
 * flush the queue) and the PackedSparseAttentionIndexer commit message
 * quoted on the "[WebGPU] Implement SparseAttentionIndexer" page
 * ("Description": packed metadata validated on the device, without host
 * synchronisation, in the normal provider paths).  This library's reading:
 * the hot-path entry points never read metadata back and never synchronise;
 * they trust it and check only host-known sizes.  The full check of the
 * device arrays is this separate call, for tests and debugging, and it is
 * the one entry point that synchronises.
 *
 * Copies the arrays to the host (synchronising `stream`) and writes a bit
 * mask of violations to *violations (host pointer):
 *   bit 0 cu_seqlens_q[0] != 0        bit 1 cu_seqlens_q decreasing
 *   bit 2 cu_seqlens_q[num_seqs] != num_tokens
 *   bit 3 seqlens_kv[b] < q_len_b     bit 4 seqlens_kv[b] beyond the table row
 *   bit 5 a needed block id outside [0, num_blocks)
 *   bit 6 a slot >= num_blocks * block_size
 *   bit 7 duplicate non-negative slots
 * slot_mapping may be NULL (bits 6-7 then stay clear).  Returns PA_OK when
 * the check ran, whatever it found.
 */
pa_status_t pa_validate_metadata(const int32_t* cu_seqlens_q,
                                 const int32_t* seqlens_kv,
                                 const int32_t* block_table,
                                 const int32_t* slot_mapping, int32_t num_seqs,
                                 int64_t num_tokens, int32_t max_blocks_per_seq,
                                 int64_t num_blocks, int32_t block_size,
                                 uint32_t* violations, void* stream);

/* Human-readable name of a status code (static storage): the names of the
 * pa_status_t convention above ("[WebGPU] Initial PagedAttention
 * implementation (1/n)", "Description" and the review rounds' cache-output
 * aliasing contract); "PA_ERR_UNKNOWN" for any other value. */
const char* pa_status_string(int32_t status);

/* Message describing the calling thread's most recent failed call
 * (static thread-local storage; "" if none). */
const char* pa_last_error(void);

/*
 * Kernel timing for measurement tools.  While enabled, the scatter and
 * attention entry points bracket each kernel launch with a pair of HIP
 * events on the caller's stream.  pa_profile_read waits for the recorded
 * events and returns, per kernel kind, the summed milliseconds and launch
 * counts (host arrays of n entries; kinds: 0 scatter (all three scatter
 * entry points), 1 plan (and pa_seqlens_from_past), 2 attention (the one
 * launch that runs prefill tiles and split-KV decode items; the fp8 launch
 * of pa_attention_fp8), 3 split-KV combine, 4 pa_rotary_scatter_kv), then
 * forgets them.  Not for concurrent use.
 */
#define PA_PROFILE_KINDS 5
pa_status_t pa_profile_enable(int32_t enable);
pa_status_t pa_profile_read(double* ms, int64_t* launches, int32_t n);
/* Which kinds profiling brackets with events: bit k of kind_mask selects
 * kind k (default: every kind).  Launches of other kinds get no events, so
 * a measurement that needs one kernel's duration adds nothing around the
 * rest.  Bits from PA_PROFILE_KINDS up are ignored. */
pa_status_t pa_profile_select(uint32_t kind_mask);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
