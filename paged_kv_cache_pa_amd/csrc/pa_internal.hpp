// Internal (non-ABI) declarations shared by the host entry points and the
// kernel translation units: work-partition constants, the workspace layout
// and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Split-KV length of the decode path (keys per work item).  A sequence's
// split depends on nothing but this length, so its output never depends on
// its batch-mates.  1024 measured faster than 512 on the large mixed batch
// (half the split partials to write and combine) and the same on pure
// decode; 256 was 7 % slower (per-item start-up), and 2048 no faster on
// the mixed batch (a cheaper combine, longer decode items).  The kernels
// take the length as an argument (a power of two, at most 128 blocks: two
// registers of block ids, one per lane each), so a test-only host override
// can vary it.
constexpr int kSplitKeys = 1024;
// Largest split count per sequence (the block table row bounds the context:
// max_blocks_per_seq * block_size <= kSplitKeys * kMaxSplitsCombine).
constexpr int kMaxSplitsCombine = 256;
// A sequence takes the decode path when q_len * G columns fit one 16-wide
// matrix-core tile.
constexpr int kDecodeCols = 16;
// Prefill tile: 256 (token, head-in-group) rows per work-group (8 waves of
// 32 rows), 64 keys per K/V tile.
constexpr int kPrefillRows = 256;
constexpr int kPrefillKeys = 64;
constexpr int kQueues = 8;  // one prefill work queue per XCD
// Cost model of the attention kernel's role split: one prefill tile step
// (256 query rows x 64 keys) is weighed as this many decode key rows (K and
// V of one KV head); both scale with head_size.  Per-CU measurements on
// MI355X (2.8 us per bf16/fp16 tile step at head_size 128, 13.5 ns per
// 512-byte key row with ~96 CUs streaming) put it near 200; with the
// current decode loads an A/B on the large mixed batch settled on 160
// (0.8 % faster than 200, in each of 4 interleaved reps; 250 was 1 %
// slower).  Only batches with both kinds of sequence depend on it.
constexpr float kPrefillStepCost = 160.f;
constexpr int kMaxGroup = 128;  // largest supported num_heads / num_kv_heads
// Largest count of decode items, prefill items or split-KV partial rows a
// call may produce: these are 32-bit on the device, and the fetch counters
// run past the item count by at most one per wave.
constexpr int kMaxWorkItems = 1 << 30;
constexpr float kLog2e = 1.4426950408889634f;

// Counter block at the start of the workspace (int32 slots).  Every fetch
// counter (a device-scope atomic) has a 128-byte cache line of its own, and
// the read-only plan results share another: atomics on a line serialize at
// the L2, so reads or atomics that shared a line with the decode counter
// would queue behind its traffic and hold up the decode item fetches.
constexpr int kLine = 32;   // int32 slots per 128-byte line
enum Counter : int {
  kCtrDecode = 0,                          // decode work fetch counter
  kCtrPrefill = kLine,                     // + kLine * x: fetch counter of prefill queue x
  kPlanResults = kLine * (1 + kQueues),    // read-only plan results from here:
  kNumDecPairs = kPlanResults,             //   number of (sequence, split) decode pairs
  kQueueLen = kPlanResults + 1,            //   + x: items in prefill queue x
  kQueueStart = kPlanResults + 1 + kQueues,  // + x: first item of queue x
  kPrefillFirst = kPlanResults + 1 + 2 * kQueues,  // attention groups [0, this) start on prefill
  kNumCounters = kPlanResults + kLine
};
static_assert(kPrefillFirst < kNumCounters, "counter block layout");

struct SeqInfo {  // one per sequence, written by the plan kernel
  int32_t cu;     // first packed token
  int32_t q_len;
  int32_t kv_len;
  int32_t pbase;  // first split-KV partial row (decode path, nsplit > 1)
};

struct Layout {
  size_t counters, seqinfo, dec_items, pf_items, part_ml, part_acc, total;
  int64_t max_dec_pairs, max_pf_items, max_part_rows;
};

struct Shape {
  int32_t num_seqs;
  int64_t num_tokens;
  int32_t max_blocks_per_seq;
  int32_t num_heads, num_kv_heads, head_size, block_size;
  int32_t split_keys;   // decode split length (kSplitKeys unless overridden for tests)
};

// Tokens per prefill tile for a GQA group size.
inline int prefill_tokens_per_tile(int group) { return kPrefillRows / group; }

Layout workspace_layout(const Shape& s);

struct PlanArgs {
  const int32_t* cu_seqlens_q;
  const int32_t* seqlens_kv;
  int32_t* counters;
  SeqInfo* seqinfo;
  int2* dec_items;
  int4* pf_items;
  int32_t num_seqs, group, num_kv_heads, tokens_per_tile;
  int32_t num_workers;  // grid size of the attention kernel
  int32_t decode_only;  // fp8 caches: only the decode path; a sequence with
                        // more than kDecodeCols columns gets no work items
  int32_t window;       // local_window_size (0: off)
  int32_t split_keys, split_shift;   // decode split length and its log2
  int32_t force_prefill;             // every sequence takes the prefill path (test override)
};

struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  void* out;
  const int32_t* block_table;
  const int32_t* counters;
  int32_t* counters_rw;
  const SeqInfo* seqinfo;
  const int2* dec_items;
  const int4* pf_items;
  float2* part_ml;
  float* part_acc;
  const float* k_scale;   // fp8 caches: [num_kv_heads, head_size] float32
  const float* v_scale;
  int32_t num_seqs, num_heads, num_kv_heads, group, max_blocks_per_seq;
  int32_t block_size, block_shift, tokens_per_tile;
  float scale_log2;  // scale * log2(e)
  float inv_group;   // 1 / group (exact small-integer division, see div_small)
  // Score soft cap c > 0: capped score in log2 units = cap_b - 2 cap_b /
  // (2^(s * cap_k) + 1) = c tanh(scale s / c) log2(e) for the raw dot product
  // s, with cap_k = 2 (scale / c) log2(e) and cap_b = c log2(e); cap_b = 0: off.
  float cap_k, cap_b;
  int32_t window;    // local_window_size W: row sees keys (limit - W, limit]; 0: off
  int32_t split_keys, split_shift;   // decode split length and its log2
  int32_t force_prefill;             // no sequence took the decode path (test override)
  // Q rows: element (t, h, d) at q[t * q_stride + h * head_size + d]
  // (q_stride = num_heads * head_size, or the packed QKV row).  rope_dim > 0:
  // Q is rotated as it is loaded (rope_chunk) at its token's position, which
  // must be below rope_max_pos (other rows are used unrotated).
  int64_t q_stride;
  const void* rope_cos;   // [rope_max_pos, rope_dim / 2] dtype
  const void* rope_sin;
  int32_t rope_dim, rope_inter, rope_max_pos;
};

// First decode split of a sequence with a sliding window: splits wholly
// below the window start of its first new row hold no visible key.
__host__ __device__ inline int first_live_split(int kv_len, int q_len, int window,
                                                int split_shift) {
  if (window <= 0) return 0;
  const int lo = kv_len - q_len - window + 1;   // first visible key of row 0
  return lo > 0 ? lo >> split_shift : 0;
}

hipError_t launch_scatter(const void* k_new, const void* v_new, const int32_t* slots, void* kc,
                          void* vc, int64_t num_tokens, int32_t row_bytes, hipStream_t st);
hipError_t launch_scatter_fp8(const void* k_new, const void* v_new, const int32_t* slots,
                              const float* k_scale, const float* v_scale, void* kc, void* vc,
                              int64_t num_tokens, int32_t row_elems, int32_t dtype,
                              hipStream_t st);
// kv8: fp8 caches (codes quantized with k_scale / v_scale); otherwise the
// scales are unused and the rows are copied.
hipError_t launch_scatter_paged(const void* k_new, const void* v_new, const int32_t* cu,
                                const int32_t* lens, const int32_t* table, void* kc, void* vc,
                                const float* k_scale, const float* v_scale, int32_t num_seqs,
                                int64_t num_tokens, int32_t max_blocks, int32_t block_size,
                                int32_t row_elems, int32_t dtype, bool kv8, hipStream_t st);
// Rotary embedding + packed-QKV split + scatter of one batch of new tokens.
struct RotaryArgs {
  const void* query;      // [T, Hq, D], or packed [T, Hq + 2 Hk, D] when key is null
  const void* key;        // [T, Hk, D] or null
  const void* value;      // [T, Hk, D] or null
  const void* cos_cache;  // [max_position, rotary_dim / 2] or null (no rotation)
  const void* sin_cache;
  const int32_t* cu;
  const int32_t* lens;
  const int32_t* table;
  void* q_out;            // [T, Hq, D], or null (Q rows skipped)
  void* k_cache;          // [NB, bs, Hk, D] dtype, or uint8 e4m3 codes with k_scale
  void* v_cache;
  const float* k_scale;   // fp8 caches: [Hk, D] float32 per-channel scales; else null
  const float* v_scale;
  int64_t num_tokens;
  int32_t num_seqs, max_blocks, block_size;
  int32_t num_heads, num_kv_heads, head_size;
  int32_t max_position, rotary_dim, interleaved;
};
hipError_t launch_rotary_scatter(const RotaryArgs& a, int dtype, hipStream_t st);
hipError_t launch_seqlens_from_past(const int32_t* cu, const int32_t* past, int32_t* out,
                                    int32_t num_seqs, hipStream_t st);
hipError_t launch_plan(const PlanArgs& a, hipStream_t st);
// The attention kernel is persistent: one 512-thread work-group per slot the
// device holds at once.  Work-groups [0, counters[kPrefillFirst]) run prefill
// items first and then decode items; the others run decode items first, so
// compute-bound prefill and bandwidth-bound decode overlap across CUs.
// kv8: the kernel for fp8 caches, which runs decode items only.
int attention_workers(int dtype, int head_size, int num_cus, bool kv8 = false);
hipError_t launch_attention(const AttnArgs& a, int dtype, int head_size, int grid,
                            hipStream_t st, bool kv8 = false);
hipError_t launch_combine(const AttnArgs& a, int dtype, int head_size, hipStream_t st);

// Work-groups of `kernel` (`threads` per group) resident at once.
int resident_blocks(const void* kernel, int num_cus, int threads = 256);

}  // namespace pa
