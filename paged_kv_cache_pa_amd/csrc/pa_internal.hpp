// Internal (non-ABI) declarations shared by the host entry points and the
// kernel translation units: work-partition constants, the workspace layout
// and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Split-KV length of the decode path (keys per work item).  It depends on
// nothing but this constant, so a sequence's output never depends on its
// batch-mates.
constexpr int kSplitKeys = 512;
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
constexpr int kMaxGroup = 128;  // largest supported num_heads / num_kv_heads
constexpr float kLog2e = 1.4426950408889634f;

// Counter block at the start of the workspace (int32 slots).
enum Counter : int {
  kCtrDecode = 0,            // decode work fetch counter
  kCtrPrefill = 1,           // 1..8: per-queue prefill fetch counters
  kNumDecPairs = 9,          // number of (sequence, split) decode pairs
  kQueueLen = 10,            // 10..17
  kQueueStart = 18,          // 18..25
  kNumCounters = 64
};

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
  int32_t num_seqs, num_heads, num_kv_heads, group, max_blocks_per_seq;
  int32_t block_size, block_shift, tokens_per_tile;
  float scale_log2;  // scale * log2(e)
};

hipError_t launch_scatter(const void* k_new, const void* v_new, const int32_t* slots, void* kc,
                          void* vc, int64_t num_tokens, int32_t row_bytes, hipStream_t st);
hipError_t launch_plan(const PlanArgs& a, hipStream_t st);
// Persistent kernels: the launchers size the grid as min(what the device
// holds at once, max_blocks) so no work-group is launched only to exit.
hipError_t launch_decode(const AttnArgs& a, int dtype, int head_size, int64_t max_blocks,
                         int num_cus, hipStream_t st);
hipError_t launch_combine(const AttnArgs& a, int dtype, int head_size, hipStream_t st);
hipError_t launch_prefill(const AttnArgs& a, int dtype, int head_size, int64_t max_blocks,
                          int num_cus, hipStream_t st);

// Work-groups of `kernel` (`threads` per group) resident at once.
int resident_blocks(const void* kernel, int num_cus, int threads = 256);

}  // namespace pa
