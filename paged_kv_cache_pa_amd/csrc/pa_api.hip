// Host side of the C ABI declared in include/pa.h: argument checks (all
// before the first HIP call), workspace layout, grid sizing from host-known
// bounds, kernel launches on the caller's stream, metadata validation and
// per-kernel event timing.
//
// Sources for the checks: "[WebGPU] Initial PagedAttention implementation
// (1/n)" - "Description" (unsupported features are rejected up front with a
// NOT_IMPLEMENTED status), the review's cross-cutting point on the blocking
// metadata readback (nothing here reads device metadata on the host, except
// the debug validator), and the FlexAttention page's requirement that the
// query head count be a multiple of the KV head count.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <vector>

#include "../../include/pa.h"
#include "pa_internal.hpp"

namespace {

thread_local char g_err[512] = "";

pa_status_t fail(pa_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pa_status_t fail(pa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

pa_status_t hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int64_t x) {
  int s = 0;
  while ((int64_t(1) << s) < x) ++s;
  return s;
}

// ---------------------------------------------------------------- profiling
struct ProfEvent {
  int kind;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
uint32_t g_prof_mask = ~0u;   // kinds bracketed while profiling is on
std::vector<ProfEvent> g_prof_pending;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` on `st`, bracketed by timing events while profiling is on.
template <typename F>
hipError_t timed(int kind, hipStream_t st, F&& launch) {
  if (!g_prof_on || !((g_prof_mask >> kind) & 1u)) return launch();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfEvent pe{kind, prof_event(), prof_event()};
  if (pe.start) (void)hipEventRecord(pe.start, st);
  hipError_t e = launch();
  if (pe.stop) (void)hipEventRecord(pe.stop, st);
  if (pe.start && pe.stop) g_prof_pending.push_back(pe);
  return e;
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Test-only overrides, read once per process from the environment and not
// part of the ABI: PA_TEST_SPLIT_KEYS (256, 512, 1024 or 2048: the decode
// split length) and PA_TEST_PATH=prefill (every sequence takes the prefill
// path, including those whose q_len * G fits one decode tile).  Tests vary
// them to demand the same results under other tile and split parameters.
struct TestOverrides {
  int split_keys = pa::kSplitKeys;
  bool force_prefill = false;
  bool valid = true;
  char msg[160] = "";
};
const TestOverrides& test_overrides() {
  static TestOverrides o;
  static std::once_flag once;
  std::call_once(once, [] {
    if (const char* v = getenv("PA_TEST_SPLIT_KEYS")) {
      const int k = atoi(v);
      if (k == 256 || k == 512 || k == 1024 || k == 2048) {
        o.split_keys = k;
      } else {
        o.valid = false;
        snprintf(o.msg, sizeof(o.msg), "PA_TEST_SPLIT_KEYS=%s (test override): 256, 512, 1024 or 2048", v);
      }
    }
    if (const char* v = getenv("PA_TEST_PATH")) {
      if (strcmp(v, "prefill") == 0) {
        o.force_prefill = true;
      } else if (strcmp(v, "auto") != 0) {
        o.valid = false;
        snprintf(o.msg, sizeof(o.msg), "PA_TEST_PATH=%s (test override): prefill or auto", v);
      }
    }
  });
  return o;
}

pa::Shape make_shape(int32_t num_seqs, int64_t num_tokens, int32_t max_blocks_per_seq,
                     int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                     int32_t block_size) {
  return pa::Shape{num_seqs, num_tokens, max_blocks_per_seq, num_heads, num_kv_heads, head_size,
                   block_size, test_overrides().split_keys};
}

// Host-side shape checks shared by pa_attention and the workspace query.
pa_status_t check_shape(const pa::Shape& s) {
  if (!test_overrides().valid) return fail(PA_ERR_INVALID_ARGUMENT, "%s", test_overrides().msg);
  if (s.num_seqs < 1 || s.num_seqs > 65536)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs=%d outside [1, 65536]", s.num_seqs);
  if (s.num_tokens < 0 || s.num_tokens > INT32_MAX)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_tokens=%lld outside [0, INT32_MAX]",
                (long long)s.num_tokens);
  if (s.max_blocks_per_seq < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq=%d < 1", s.max_blocks_per_seq);
  if (s.num_heads < 1 || s.num_kv_heads < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "head counts must be >= 1");
  if (s.num_heads % s.num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_heads=%d is not a multiple of num_kv_heads=%d",
                s.num_heads, s.num_kv_heads);
  if (s.num_heads / s.num_kv_heads > pa::kMaxGroup)
    return fail(PA_ERR_NOT_IMPLEMENTED, "group size %d > %d", s.num_heads / s.num_kv_heads,
                pa::kMaxGroup);
  if (s.head_size != 64 && s.head_size != 128)
    return fail(PA_ERR_NOT_IMPLEMENTED, "head_size=%d (supported: 64, 128)", s.head_size);
  if (!is_pow2(s.block_size) || s.block_size < 16 || s.block_size > 1024)
    return fail(PA_ERR_NOT_IMPLEMENTED, "block_size=%d (supported: powers of two in [16, 1024])",
                s.block_size);
  if ((int64_t)s.max_blocks_per_seq * s.block_size > (int64_t)s.split_keys * pa::kMaxSplitsCombine)
    return fail(PA_ERR_NOT_IMPLEMENTED, "max_blocks_per_seq * block_size exceeds %d tokens",
                s.split_keys * pa::kMaxSplitsCombine);
  if (s.split_keys > 128 * s.block_size)   // a decode split's block ids fill two registers
    return fail(PA_ERR_NOT_IMPLEMENTED, "split length %d exceeds 128 blocks of %d", s.split_keys,
                s.block_size);
  // The kernels' 32-bit quantities: a prefill lane's byte offset inside a
  // cache block, and the work-item, queue and partial-row counts the plan
  // writes and the fetch counters run past by at most one per wave.
  if ((int64_t)s.block_size * s.num_kv_heads * s.head_size * 2 > INT32_MAX)
    return fail(PA_ERR_NOT_IMPLEMENTED, "block_size * num_kv_heads * head_size * 2 bytes exceed "
                "INT32_MAX");
  const pa::Layout L = pa::workspace_layout(s);
  if (L.max_dec_pairs * s.num_kv_heads > pa::kMaxWorkItems || L.max_pf_items > pa::kMaxWorkItems ||
      L.max_part_rows > pa::kMaxWorkItems)
    return fail(PA_ERR_NOT_IMPLEMENTED, "work items or split-KV partial rows exceed %d "
                "(decode items %lld, prefill items %lld, partial rows %lld)", pa::kMaxWorkItems,
                (long long)(L.max_dec_pairs * s.num_kv_heads), (long long)L.max_pf_items,
                (long long)L.max_part_rows);
  return PA_OK;
}

bool aligned16(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (((uintptr_t)p & 15) != 0) return false;
  return true;
}

}  // namespace

namespace pa {

int resident_blocks(const void* kernel, int num_cus, int threads) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  return per_cu * num_cus;
}

Layout workspace_layout(const Shape& s) {
  Layout L{};
  const int G = s.num_heads / s.num_kv_heads;
  const int64_t max_kv = (int64_t)s.max_blocks_per_seq * s.block_size;
  const int64_t max_splits = (max_kv + s.split_keys - 1) / s.split_keys;
  const int tq = prefill_tokens_per_tile(G);
  L.max_dec_pairs = (int64_t)s.num_seqs * max_splits;
  const int64_t cols = std::min<int64_t>((int64_t)kDecodeCols * s.num_seqs, (int64_t)G * s.num_tokens);
  L.max_part_rows = max_splits > 1 ? max_splits * s.num_kv_heads * cols : 0;
  L.max_pf_items = ((s.num_tokens + tq - 1) / tq + std::min<int64_t>(s.num_seqs, s.num_tokens)) *
                   s.num_kv_heads;
  size_t off = 0;
  L.counters = off;
  off = align256(off + kNumCounters * sizeof(int32_t));
  L.seqinfo = off;
  off = align256(off + (size_t)s.num_seqs * sizeof(SeqInfo));
  L.dec_items = off;
  off = align256(off + (size_t)L.max_dec_pairs * sizeof(int2));
  L.pf_items = off;
  off = align256(off + (size_t)L.max_pf_items * sizeof(int4));
  L.part_ml = off;
  off = align256(off + (size_t)L.max_part_rows * sizeof(float2));
  L.part_acc = off;
  off = align256(off + (size_t)L.max_part_rows * s.head_size * sizeof(float));
  L.total = off;
  return L;
}

}  // namespace pa

extern "C" {

const char* pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARGUMENT: return "PA_ERR_INVALID_ARGUMENT";
    case PA_ERR_NOT_IMPLEMENTED: return "PA_ERR_NOT_IMPLEMENTED";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    default: return "PA_ERR_UNKNOWN";
  }
}

const char* pa_last_error(void) { return g_err; }

pa_status_t pa_scatter_kv(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                          void* k_cache, void* v_cache, int64_t num_tokens, int64_t num_blocks,
                          int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                          int32_t dtype, void* stream) {
  g_err[0] = 0;
  if (dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_NOT_IMPLEMENTED, "dtype=%d (supported: PA_F16, PA_BF16)", dtype);
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_tokens < 0");
  if (num_kv_heads < 1 || head_size < 1 || block_size < 1 || num_blocks < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "sizes must be >= 1");
  if (head_size % 8 != 0)
    return fail(PA_ERR_NOT_IMPLEMENTED, "head_size=%d is not a multiple of 8", head_size);
  if (num_blocks * (int64_t)block_size > INT32_MAX)
    return fail(PA_ERR_NOT_IMPLEMENTED, "num_blocks * block_size exceeds INT32_MAX");
  const int64_t row_bytes = (int64_t)num_kv_heads * head_size * 2;
  if (row_bytes > INT32_MAX) return fail(PA_ERR_NOT_IMPLEMENTED, "row too large");
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache)
    return fail(PA_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (!aligned16({k_new, v_new, k_cache, v_cache}))
    return fail(PA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed(0, st, [&] {
    return pa::launch_scatter(k_new, v_new, slot_mapping, k_cache, v_cache, num_tokens,
                              (int32_t)row_bytes, st);
  });
  if (e != hipSuccess) return hip_fail(e, "scatter launch");
  return PA_OK;
}

pa_status_t pa_scatter_kv_fp8(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                              const float* k_scale, const float* v_scale, void* k_cache,
                              void* v_cache, int64_t num_tokens, int64_t num_blocks,
                              int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                              int32_t dtype, void* stream) {
  g_err[0] = 0;
  if (dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_NOT_IMPLEMENTED, "dtype=%d (supported: PA_F16, PA_BF16)", dtype);
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_tokens < 0");
  if (num_kv_heads < 1 || head_size < 1 || block_size < 1 || num_blocks < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "sizes must be >= 1");
  if (head_size % 8 != 0)
    return fail(PA_ERR_NOT_IMPLEMENTED, "head_size=%d is not a multiple of 8", head_size);
  if (num_blocks * (int64_t)block_size > INT32_MAX)
    return fail(PA_ERR_NOT_IMPLEMENTED, "num_blocks * block_size exceeds INT32_MAX");
  const int64_t row_elems = (int64_t)num_kv_heads * head_size;
  if (row_elems * 2 > INT32_MAX) return fail(PA_ERR_NOT_IMPLEMENTED, "row too large");
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_scale || !v_scale || !k_cache || !v_cache)
    return fail(PA_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (!aligned16({k_new, v_new, k_scale, v_scale, k_cache, v_cache}))
    return fail(PA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed(0, st, [&] {
    return pa::launch_scatter_fp8(k_new, v_new, slot_mapping, k_scale, v_scale, k_cache, v_cache,
                                  num_tokens, (int32_t)row_elems, dtype, st);
  });
  if (e != hipSuccess) return hip_fail(e, "fp8 scatter launch");
  return PA_OK;
}

static pa_status_t scatter_paged_impl(const void* k_new, const void* v_new,
                                      const int32_t* cu_seqlens_q, const int32_t* seqlens_kv,
                                      const int32_t* block_table, const float* k_scale,
                                      const float* v_scale, void* k_cache, void* v_cache,
                                      int32_t num_seqs, int64_t num_tokens,
                                      int32_t max_blocks_per_seq, int64_t num_blocks,
                                      int32_t num_kv_heads, int32_t head_size,
                                      int32_t block_size, int32_t dtype, void* stream, bool kv8) {
  if (dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_NOT_IMPLEMENTED, "dtype=%d (supported: PA_F16, PA_BF16)", dtype);
  if (num_tokens < 0 || num_tokens > INT32_MAX)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_tokens outside [0, INT32_MAX]");
  if (num_seqs < 1 || max_blocks_per_seq < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs and max_blocks_per_seq must be >= 1");
  if (num_kv_heads < 1 || head_size < 1 || block_size < 1 || num_blocks < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "sizes must be >= 1");
  if (head_size % 8 != 0)
    return fail(PA_ERR_NOT_IMPLEMENTED, "head_size=%d is not a multiple of 8", head_size);
  if (num_blocks * (int64_t)block_size > INT32_MAX)
    return fail(PA_ERR_NOT_IMPLEMENTED, "num_blocks * block_size exceeds INT32_MAX");
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX)
    return fail(PA_ERR_NOT_IMPLEMENTED, "max_blocks_per_seq * block_size exceeds INT32_MAX");
  const int64_t row_elems = (int64_t)num_kv_heads * head_size;
  if (row_elems * 2 > INT32_MAX) return fail(PA_ERR_NOT_IMPLEMENTED, "row too large");
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !cu_seqlens_q || !seqlens_kv || !block_table || !k_cache || !v_cache)
    return fail(PA_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (kv8 && (!k_scale || !v_scale)) return fail(PA_ERR_INVALID_ARGUMENT, "null scale pointer");
  if (!aligned16({k_new, v_new, k_cache, v_cache}) || (kv8 && !aligned16({k_scale, v_scale})))
    return fail(PA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed(0, st, [&] {
    return pa::launch_scatter_paged(k_new, v_new, cu_seqlens_q, seqlens_kv, block_table, k_cache,
                                    v_cache, k_scale, v_scale, num_seqs, num_tokens,
                                    max_blocks_per_seq, block_size, (int32_t)row_elems, dtype,
                                    kv8, st);
  });
  if (e != hipSuccess) return hip_fail(e, "scatter launch");
  return PA_OK;
}

pa_status_t pa_scatter_kv_paged(const void* k_new, const void* v_new, const int32_t* cu_seqlens_q,
                                const int32_t* seqlens_kv, const int32_t* block_table,
                                void* k_cache, void* v_cache, int32_t num_seqs,
                                int64_t num_tokens, int32_t max_blocks_per_seq, int64_t num_blocks,
                                int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                int32_t dtype, void* stream) {
  g_err[0] = 0;
  return scatter_paged_impl(k_new, v_new, cu_seqlens_q, seqlens_kv, block_table, nullptr, nullptr,
                            k_cache, v_cache, num_seqs, num_tokens, max_blocks_per_seq, num_blocks,
                            num_kv_heads, head_size, block_size, dtype, stream, false);
}

pa_status_t pa_scatter_kv_paged_fp8(const void* k_new, const void* v_new,
                                    const int32_t* cu_seqlens_q, const int32_t* seqlens_kv,
                                    const int32_t* block_table, const float* k_scale,
                                    const float* v_scale, void* k_cache, void* v_cache,
                                    int32_t num_seqs, int64_t num_tokens,
                                    int32_t max_blocks_per_seq, int64_t num_blocks,
                                    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                    int32_t dtype, void* stream) {
  g_err[0] = 0;
  return scatter_paged_impl(k_new, v_new, cu_seqlens_q, seqlens_kv, block_table, k_scale, v_scale,
                            k_cache, v_cache, num_seqs, num_tokens, max_blocks_per_seq, num_blocks,
                            num_kv_heads, head_size, block_size, dtype, stream, true);
}

static pa_status_t rotary_impl(const void* query, const void* key, const void* value,
                               const void* cos_cache, const void* sin_cache, int32_t max_position,
                               int32_t rotary_dim, int32_t interleaved,
                               const int32_t* cu_seqlens_q, const int32_t* seqlens_kv,
                               const int32_t* block_table, const float* k_scale,
                               const float* v_scale, void* q_out, void* k_cache, void* v_cache,
                               int32_t num_seqs, int64_t num_tokens, int32_t max_blocks_per_seq,
                               int64_t num_blocks, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_size, int32_t block_size, int32_t dtype, void* stream,
                               bool kv8) {
  if (dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_NOT_IMPLEMENTED, "dtype=%d (supported: PA_F16, PA_BF16)", dtype);
  if (num_tokens < 0 || num_tokens > INT32_MAX)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_tokens outside [0, INT32_MAX]");
  if (num_seqs < 1 || max_blocks_per_seq < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs and max_blocks_per_seq must be >= 1");
  if (num_heads < 1 || num_kv_heads < 1 || head_size < 1 || block_size < 1 || num_blocks < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "sizes must be >= 1");
  if (head_size % 8 != 0)
    return fail(PA_ERR_NOT_IMPLEMENTED, "head_size=%d is not a multiple of 8", head_size);
  if (num_blocks * (int64_t)block_size > INT32_MAX)
    return fail(PA_ERR_NOT_IMPLEMENTED, "num_blocks * block_size exceeds INT32_MAX");
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX)
    return fail(PA_ERR_NOT_IMPLEMENTED, "max_blocks_per_seq * block_size exceeds INT32_MAX");
  if ((key == nullptr) != (value == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "key and value must both be given or both be null");
  if ((cos_cache == nullptr) != (sin_cache == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "cos_cache and sin_cache must both be given or both be null");
  const bool rot = cos_cache != nullptr;
  if (rot) {
    if (rotary_dim < 1 || rotary_dim > head_size)
      return fail(PA_ERR_INVALID_ARGUMENT, "rotary_dim=%d outside [1, head_size]", rotary_dim);
    if (rotary_dim % 16 != 0)
      return fail(PA_ERR_NOT_IMPLEMENTED, "rotary_dim=%d is not a multiple of 16", rotary_dim);
    if (max_position < 1) return fail(PA_ERR_INVALID_ARGUMENT, "max_position < 1");
  }
  if (num_tokens == 0) return PA_OK;
  if (!cu_seqlens_q || !seqlens_kv || !block_table || !k_cache || !v_cache)
    return fail(PA_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (kv8 && (!k_scale || !v_scale)) return fail(PA_ERR_INVALID_ARGUMENT, "null scale pointer");
  // Q is neither read nor written when q_out is null and K, V come apart.
  if (!query && (q_out || !key))
    return fail(PA_ERR_INVALID_ARGUMENT, "null query (allowed only with separate key/value and no q_out)");
  for (const void* ptr : {query, key, value, cos_cache, sin_cache, (const void*)q_out,
                          (const void*)k_cache, (const void*)v_cache, (const void*)k_scale,
                          (const void*)v_scale})
    if (((uintptr_t)ptr & 15) != 0)
      return fail(PA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  pa::RotaryArgs a{};
  a.query = query;
  a.key = key;
  a.value = value;
  a.cos_cache = cos_cache;
  a.sin_cache = sin_cache;
  a.cu = cu_seqlens_q;
  a.lens = seqlens_kv;
  a.table = block_table;
  a.q_out = q_out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = kv8 ? k_scale : nullptr;
  a.v_scale = kv8 ? v_scale : nullptr;
  a.num_tokens = num_tokens;
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.block_size = block_size;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_size = head_size;
  a.max_position = rot ? max_position : 0;
  a.rotary_dim = rot ? rotary_dim : 0;
  a.interleaved = interleaved ? 1 : 0;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed(4, st, [&] { return pa::launch_rotary_scatter(a, dtype, st); });
  if (e != hipSuccess) return hip_fail(e, "rotary scatter launch");
  return PA_OK;
}

pa_status_t pa_rotary_scatter_kv(const void* query, const void* key, const void* value,
                                const void* cos_cache, const void* sin_cache,
                                int32_t max_position, int32_t rotary_dim, int32_t interleaved,
                                const int32_t* cu_seqlens_q, const int32_t* seqlens_kv,
                                const int32_t* block_table, void* q_out, void* k_cache,
                                void* v_cache, int32_t num_seqs, int64_t num_tokens,
                                int32_t max_blocks_per_seq, int64_t num_blocks, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                int32_t dtype, void* stream) {
  g_err[0] = 0;
  return rotary_impl(query, key, value, cos_cache, sin_cache, max_position, rotary_dim,
                     interleaved, cu_seqlens_q, seqlens_kv, block_table, nullptr, nullptr, q_out,
                     k_cache, v_cache, num_seqs, num_tokens, max_blocks_per_seq, num_blocks,
                     num_heads, num_kv_heads, head_size, block_size, dtype, stream, false);
}

pa_status_t pa_rotary_scatter_kv_fp8(const void* query, const void* key, const void* value,
                                    const void* cos_cache, const void* sin_cache,
                                    int32_t max_position, int32_t rotary_dim,
                                    int32_t interleaved, const int32_t* cu_seqlens_q,
                                    const int32_t* seqlens_kv, const int32_t* block_table,
                                    const float* k_scale, const float* v_scale, void* q_out,
                                    void* k_cache, void* v_cache, int32_t num_seqs,
                                    int64_t num_tokens, int32_t max_blocks_per_seq,
                                    int64_t num_blocks, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_size, int32_t block_size, int32_t dtype,
                                    void* stream) {
  g_err[0] = 0;
  return rotary_impl(query, key, value, cos_cache, sin_cache, max_position, rotary_dim,
                     interleaved, cu_seqlens_q, seqlens_kv, block_table, k_scale, v_scale, q_out,
                     k_cache, v_cache, num_seqs, num_tokens, max_blocks_per_seq, num_blocks,
                     num_heads, num_kv_heads, head_size, block_size, dtype, stream, true);
}

pa_status_t pa_seqlens_from_past(const int32_t* cu_seqlens_q, const int32_t* past_seqlens,
                                 int32_t* seqlens_kv, int32_t num_seqs, void* stream) {
  g_err[0] = 0;
  if (num_seqs < 1) return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs < 1");
  if (!cu_seqlens_q || !past_seqlens || !seqlens_kv)
    return fail(PA_ERR_INVALID_ARGUMENT, "null pointer argument");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed(1, st, [&] {
    return pa::launch_seqlens_from_past(cu_seqlens_q, past_seqlens, seqlens_kv, num_seqs, st);
  });
  if (e != hipSuccess) return hip_fail(e, "lengths launch");
  return PA_OK;
}

size_t pa_attention_workspace_size(int32_t num_seqs, int64_t num_tokens, int32_t max_blocks_per_seq,
                                   int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                   int32_t block_size) {
  const pa::Shape s = make_shape(num_seqs, num_tokens, max_blocks_per_seq, num_heads,
                                 num_kv_heads, head_size, block_size);
  if (check_shape(s) != PA_OK) return 0;
  return pa::workspace_layout(s).total;
}

// Shared by pa_attention (16-bit caches) and pa_attention_fp8 (kv8: e4m3
// caches with per-channel scales, decode path only).
// Where the attention reads Q: the row stride (elements between tokens) and
// the rotary tables Q is rotated with as it is loaded (cos == nullptr: none).
struct QSource {
  int64_t row_stride;
  const void* cos;
  const void* sin;
  int32_t max_position, rotary_dim, interleaved;
};

static pa_status_t attention_impl(const void* q, const int32_t* cu_seqlens_q,
                                  const int32_t* seqlens_kv, const int32_t* block_table,
                                  const void* k_cache, const void* v_cache, const float* k_scale,
                                  const float* v_scale, void* out, int32_t num_seqs,
                                  int64_t num_tokens, int32_t max_blocks_per_seq,
                                  int64_t num_blocks, float scale, float softcap,
                                  int32_t local_window_size, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                  int32_t dtype, void* workspace, size_t workspace_bytes,
                                  void* stream, bool kv8, const QSource* qsrc = nullptr) {
  if (dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_NOT_IMPLEMENTED, "dtype=%d (supported: PA_F16, PA_BF16)", dtype);
  const pa::Shape s = make_shape(num_seqs, num_tokens, max_blocks_per_seq, num_heads,
                                 num_kv_heads, head_size, block_size);
  pa_status_t cs = check_shape(s);
  if (cs != PA_OK) return cs;
  if (num_blocks < 1) return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks < 1");
  if (num_blocks * (int64_t)block_size > INT32_MAX)
    return fail(PA_ERR_NOT_IMPLEMENTED, "num_blocks * block_size exceeds INT32_MAX");
  if (!isfinite(scale)) return fail(PA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (!(softcap >= 0.f) || !isfinite(softcap))
    return fail(PA_ERR_INVALID_ARGUMENT, "softcap must be finite and >= 0");
  // Soft-cap constants (log2 units): cap_k = 2 (scale / c) log2(e) must be a
  // finite float for the kernels' exp2 form.
  const double cap_k = softcap > 0.f ? 2.0 * ((double)scale / softcap) * (double)pa::kLog2e : 0.0;
  if (!(fabs(cap_k) <= 3.0e38))
    return fail(PA_ERR_INVALID_ARGUMENT, "softcap too small for this scale (scale / softcap overflows)");
  if (num_tokens == 0) return PA_OK;
  if (!q || !cu_seqlens_q || !seqlens_kv || !block_table || !k_cache || !v_cache || !out)
    return fail(PA_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (kv8 && (!k_scale || !v_scale)) return fail(PA_ERR_INVALID_ARGUMENT, "null scale pointer");
  if (!aligned16({q, out, k_cache, v_cache}) || (kv8 && !aligned16({k_scale, v_scale})))
    return fail(PA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  {
    // out is written while other work-groups still read q: the two must not
    // overlap (byte ranges of the rows each touches).
    const int64_t row = qsrc ? qsrc->row_stride : (int64_t)num_heads * head_size;
    const uintptr_t q0 = (uintptr_t)q, o0 = (uintptr_t)out;
    const uintptr_t q1 = q0 + (uintptr_t)(((num_tokens - 1) * row + (int64_t)num_heads * head_size) * 2);
    const uintptr_t o1 = o0 + (uintptr_t)(num_tokens * num_heads * head_size * 2);
    if (q0 < o1 && o0 < q1) return fail(PA_ERR_INVALID_ARGUMENT, "q and out overlap");
  }
  const pa::Layout L = pa::workspace_layout(s);
  if (!workspace) return fail(PA_ERR_INVALID_ARGUMENT, "null workspace");
  if (((uintptr_t)workspace & 255) != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu", workspace_bytes,
                L.total);

  char* ws = (char*)workspace;
  const int G = num_heads / num_kv_heads;
  const int tq = pa::prefill_tokens_per_tile(G);
  hipStream_t st = (hipStream_t)stream;
  const int cus = device_cus();

  pa::PlanArgs pl{};
  pl.cu_seqlens_q = cu_seqlens_q;
  pl.seqlens_kv = seqlens_kv;
  pl.counters = (int32_t*)(ws + L.counters);
  pl.seqinfo = (pa::SeqInfo*)(ws + L.seqinfo);
  pl.dec_items = (int2*)(ws + L.dec_items);
  pl.pf_items = (int4*)(ws + L.pf_items);
  pl.num_seqs = num_seqs;
  pl.group = G;
  pl.num_kv_heads = num_kv_heads;
  pl.tokens_per_tile = tq;
  pl.decode_only = kv8 ? 1 : 0;
  pl.window = local_window_size > 0 ? local_window_size : 0;
  pl.split_keys = s.split_keys;
  pl.split_shift = log2i(s.split_keys);
  pl.force_prefill = test_overrides().force_prefill && !kv8 ? 1 : 0;
  // Persistent grid: what the device holds at once, but no more groups than
  // there are prefill items plus groups of 8 decode waves.
  const int64_t max_groups =
      (kv8 ? 0 : L.max_pf_items) + (L.max_dec_pairs * num_kv_heads + 7) / 8;
  const int workers = (int)std::max<int64_t>(
      1, std::min<int64_t>(pa::attention_workers(dtype, head_size, cus, kv8), max_groups));
  pl.num_workers = workers;
  hipError_t e = timed(1, st, [&] { return pa::launch_plan(pl, st); });
  if (e != hipSuccess) return hip_fail(e, "plan launch");

  pa::AttnArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.out = out;
  a.block_table = block_table;
  a.counters = pl.counters;
  a.counters_rw = pl.counters;
  a.seqinfo = pl.seqinfo;
  a.dec_items = pl.dec_items;
  a.pf_items = pl.pf_items;
  a.part_ml = (float2*)(ws + L.part_ml);
  a.part_acc = (float*)(ws + L.part_acc);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = G;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.block_size = block_size;
  a.block_shift = log2i(block_size);
  a.tokens_per_tile = tq;
  a.scale_log2 = scale * pa::kLog2e;
  a.inv_group = 1.0f / (float)G;
  a.cap_k = (float)cap_k;
  a.cap_b = softcap > 0.f ? softcap * pa::kLog2e : 0.f;
  a.window = pl.window;
  a.split_keys = pl.split_keys;
  a.split_shift = pl.split_shift;
  a.force_prefill = pl.force_prefill;
  a.q_stride = qsrc ? qsrc->row_stride : (int64_t)num_heads * head_size;
  if (qsrc && qsrc->cos) {
    a.rope_cos = qsrc->cos;
    a.rope_sin = qsrc->sin;
    a.rope_dim = qsrc->rotary_dim;
    a.rope_inter = qsrc->interleaved ? 1 : 0;
    a.rope_max_pos = qsrc->max_position;
  }

  e = timed(2, st, [&] { return pa::launch_attention(a, dtype, head_size, workers, st, kv8); });
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  if (L.max_part_rows > 0) {
    e = timed(3, st, [&] { return pa::launch_combine(a, dtype, head_size, st); });
    if (e != hipSuccess) return hip_fail(e, "combine launch");
  }
  return PA_OK;
}

pa_status_t pa_attention(const void* q, const int32_t* cu_seqlens_q, const int32_t* seqlens_kv,
                         const int32_t* block_table, const void* k_cache, const void* v_cache,
                         void* out, int32_t num_seqs, int64_t num_tokens,
                         int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                         float softcap, int32_t local_window_size, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                         int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  return attention_impl(q, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache, nullptr,
                        nullptr, out, num_seqs, num_tokens, max_blocks_per_seq, num_blocks, scale,
                        softcap, local_window_size, num_heads, num_kv_heads, head_size, block_size, dtype, workspace,
                        workspace_bytes, stream, false);
}

// Checks of the Q-source arguments shared by pa_attention_rope and
// pa_attention_rope_fp8; fills *qs on success.
static pa_status_t rope_source(const void* cos_cache, const void* sin_cache, int32_t max_position,
                               int32_t rotary_dim, int32_t interleaved, int64_t q_row_stride,
                               int64_t num_tokens, int32_t num_heads, int32_t head_size,
                               QSource* qs) {
  if (num_heads >= 1 && head_size >= 1 && q_row_stride < (int64_t)num_heads * head_size)
    return fail(PA_ERR_INVALID_ARGUMENT, "q_row_stride=%lld < num_heads * head_size",
                (long long)q_row_stride);
  if (q_row_stride % 8 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "q_row_stride=%lld is not a multiple of 8 (16-byte rows)",
                (long long)q_row_stride);
  // The byte range of q's rows must fit 62 bits (64-bit offsets, with room).
  if (num_tokens > 0 && q_row_stride > ((int64_t)1 << 60) / num_tokens)
    return fail(PA_ERR_INVALID_ARGUMENT, "q_row_stride=%lld: q's rows exceed the address range",
                (long long)q_row_stride);
  if ((cos_cache == nullptr) != (sin_cache == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "cos_cache and sin_cache must both be given or both be null");
  if (cos_cache) {
    if (rotary_dim < 1 || rotary_dim > head_size)
      return fail(PA_ERR_INVALID_ARGUMENT, "rotary_dim=%d outside [1, head_size]", rotary_dim);
    if (rotary_dim % 16 != 0)
      return fail(PA_ERR_NOT_IMPLEMENTED, "rotary_dim=%d is not a multiple of 16", rotary_dim);
    if (max_position < 1) return fail(PA_ERR_INVALID_ARGUMENT, "max_position < 1");
    if (!aligned16({cos_cache, sin_cache}))
      return fail(PA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  }
  *qs = QSource{q_row_stride, cos_cache, sin_cache, max_position, rotary_dim, interleaved};
  return PA_OK;
}

// fp8 caches serve decode-shaped batches only: max_q_len * G within one tile.
static pa_status_t fp8_q_len_bound(int32_t max_q_len, int32_t num_heads, int32_t num_kv_heads) {
  if (max_q_len < 0) return fail(PA_ERR_INVALID_ARGUMENT, "max_q_len < 0");
  if (num_kv_heads >= 1 && num_heads >= 1 && num_heads % num_kv_heads == 0 &&
      (int64_t)max_q_len * (num_heads / num_kv_heads) > pa::kDecodeCols)
    return fail(PA_ERR_NOT_IMPLEMENTED,
                "fp8 caches: max_q_len * G = %lld exceeds %d (decode-shaped batches only)",
                (long long)max_q_len * (num_heads / num_kv_heads), pa::kDecodeCols);
  return PA_OK;
}

pa_status_t pa_attention_rope(const void* q, int64_t q_row_stride, const void* cos_cache,
                              const void* sin_cache, int32_t max_position, int32_t rotary_dim,
                              int32_t interleaved, const int32_t* cu_seqlens_q,
                              const int32_t* seqlens_kv, const int32_t* block_table,
                              const void* k_cache, const void* v_cache, void* out,
                              int32_t num_seqs, int64_t num_tokens, int32_t max_blocks_per_seq,
                              int64_t num_blocks, float scale, float softcap,
                              int32_t local_window_size, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_size, int32_t block_size, int32_t dtype,
                              void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  QSource qs{};
  const pa_status_t rs = rope_source(cos_cache, sin_cache, max_position, rotary_dim, interleaved,
                                     q_row_stride, num_tokens, num_heads, head_size, &qs);
  if (rs != PA_OK) return rs;
  return attention_impl(q, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache, nullptr,
                        nullptr, out, num_seqs, num_tokens, max_blocks_per_seq, num_blocks, scale,
                        softcap, local_window_size, num_heads, num_kv_heads, head_size,
                        block_size, dtype, workspace, workspace_bytes, stream, false, &qs);
}

pa_status_t pa_attention_rope_fp8(const void* q, int64_t q_row_stride, const void* cos_cache,
                                  const void* sin_cache, int32_t max_position,
                                  int32_t rotary_dim, int32_t interleaved,
                                  const int32_t* cu_seqlens_q, const int32_t* seqlens_kv,
                                  const int32_t* block_table, const void* k_cache,
                                  const void* v_cache, const float* k_scale,
                                  const float* v_scale, void* out, int32_t num_seqs,
                                  int64_t num_tokens, int32_t max_q_len,
                                  int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                  float softcap, int32_t local_window_size, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                  int32_t dtype, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  g_err[0] = 0;
  const pa_status_t bs = fp8_q_len_bound(max_q_len, num_heads, num_kv_heads);
  if (bs != PA_OK) return bs;
  QSource qs{};
  const pa_status_t rs = rope_source(cos_cache, sin_cache, max_position, rotary_dim, interleaved,
                                     q_row_stride, num_tokens, num_heads, head_size, &qs);
  if (rs != PA_OK) return rs;
  return attention_impl(q, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache, k_scale,
                        v_scale, out, num_seqs, num_tokens, max_blocks_per_seq, num_blocks, scale,
                        softcap, local_window_size, num_heads, num_kv_heads, head_size,
                        block_size, dtype, workspace, workspace_bytes, stream, true, &qs);
}

// ------------------------------------------------ allocation-free variant
// The fixed device scratch of pa_attention_noalloc: plan lists, counters and
// split-KV partials live here instead of in a caller workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` only names the symbol; its device address (per device) comes
// from hipGetSymbolAddress and is the only form passed to kernels.
constexpr size_t kScratchBytes = size_t(256) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}
}  // namespace

pa_status_t pa_attention_noalloc(const void* q, const int32_t* cu_seqlens_q,
                                 const int32_t* seqlens_kv, const int32_t* block_table,
                                 const void* k_cache, const void* v_cache, void* out,
                                 int32_t num_seqs, int64_t num_tokens, int32_t max_blocks_per_seq,
                                 int64_t num_blocks, float scale, float softcap,
                                 int32_t local_window_size, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                 int32_t dtype, void* stream) {
  g_err[0] = 0;
  if (dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_NOT_IMPLEMENTED, "dtype=%d (supported: PA_F16, PA_BF16)", dtype);
  // Sizes first, on the host, before any HIP call: the scratch must hold the
  // workspace pa_attention would need for these sizes.
  const pa::Shape s = make_shape(num_seqs, num_tokens, max_blocks_per_seq, num_heads,
                                 num_kv_heads, head_size, block_size);
  pa_status_t cs = check_shape(s);
  if (cs != PA_OK) return cs;
  const size_t need = pa::workspace_layout(s).total;
  if (need > kScratchBytes)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                "these sizes need %zu bytes of scratch; the fixed scratch holds %zu (use "
                "pa_attention with a caller workspace)", need, kScratchBytes);
  if (num_tokens == 0) return PA_OK;
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e, "scratch address");
  return attention_impl(q, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache, nullptr,
                        nullptr, out, num_seqs, num_tokens, max_blocks_per_seq, num_blocks, scale,
                        softcap, local_window_size, num_heads, num_kv_heads, head_size,
                        block_size, dtype, ws, kScratchBytes, stream, false);
}

pa_status_t pa_attention_fp8(const void* q, const int32_t* cu_seqlens_q,
                             const int32_t* seqlens_kv, const int32_t* block_table,
                             const void* k_cache, const void* v_cache, const float* k_scale,
                             const float* v_scale, void* out, int32_t num_seqs,
                             int64_t num_tokens, int32_t max_q_len, int32_t max_blocks_per_seq,
                             int64_t num_blocks, float scale, float softcap,
                             int32_t local_window_size, int32_t num_heads,
                             int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                             int32_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  g_err[0] = 0;
  const pa_status_t bs = fp8_q_len_bound(max_q_len, num_heads, num_kv_heads);
  if (bs != PA_OK) return bs;
  return attention_impl(q, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache, k_scale,
                        v_scale, out, num_seqs, num_tokens, max_blocks_per_seq, num_blocks, scale,
                        softcap, local_window_size, num_heads, num_kv_heads, head_size, block_size, dtype, workspace,
                        workspace_bytes, stream, true);
}

pa_status_t pa_validate_metadata(const int32_t* cu_seqlens_q, const int32_t* seqlens_kv,
                                 const int32_t* block_table, const int32_t* slot_mapping,
                                 int32_t num_seqs, int64_t num_tokens, int32_t max_blocks_per_seq,
                                 int64_t num_blocks, int32_t block_size, uint32_t* violations,
                                 void* stream) {
  g_err[0] = 0;
  if (!violations || !cu_seqlens_q || !seqlens_kv || !block_table)
    return fail(PA_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (num_seqs < 1 || num_tokens < 0 || max_blocks_per_seq < 1 || block_size < 1 || num_blocks < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "invalid sizes");
  hipStream_t st = (hipStream_t)stream;
  std::vector<int32_t> cu(num_seqs + 1), L(num_seqs), tbl((size_t)num_seqs * max_blocks_per_seq),
      slots(slot_mapping ? num_tokens : 0);
  hipError_t e = hipMemcpyAsync(cu.data(), cu_seqlens_q, cu.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(L.data(), seqlens_kv, L.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(tbl.data(), block_table, tbl.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess && slot_mapping && num_tokens > 0)
    e = hipMemcpyAsync(slots.data(), slot_mapping, slots.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "metadata copy");
  uint32_t v = 0;
  if (cu[0] != 0) v |= 1u << 0;
  for (int b = 0; b < num_seqs; ++b)
    if (cu[b + 1] < cu[b]) v |= 1u << 1;
  if (cu[num_seqs] != num_tokens) v |= 1u << 2;
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t ql = (int64_t)cu[b + 1] - cu[b];
    if (L[b] < ql) v |= 1u << 3;
    const int64_t need = ((int64_t)L[b] + block_size - 1) / block_size;
    if (need > max_blocks_per_seq) {
      v |= 1u << 4;
      continue;
    }
    for (int64_t k = 0; k < need; ++k) {
      const int32_t id = tbl[(size_t)b * max_blocks_per_seq + k];
      if (id < 0 || id >= num_blocks) v |= 1u << 5;
    }
  }
  if (slot_mapping && num_tokens > 0) {
    std::vector<int32_t> live;
    for (int32_t x : slots) {
      if (x >= (int64_t)num_blocks * block_size) v |= 1u << 6;
      if (x >= 0) live.push_back(x);
    }
    std::sort(live.begin(), live.end());
    if (std::adjacent_find(live.begin(), live.end()) != live.end()) v |= 1u << 7;
  }
  *violations = v;
  return PA_OK;
}

pa_status_t pa_profile_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = enable != 0;
  return PA_OK;
}

pa_status_t pa_profile_select(uint32_t kind_mask) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_mask = kind_mask;
  return PA_OK;
}

pa_status_t pa_profile_read(double* ms, int64_t* launches, int32_t n) {
  g_err[0] = 0;
  if (!ms || !launches || n < 1) return fail(PA_ERR_INVALID_ARGUMENT, "bad output arrays");
  for (int i = 0; i < n; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  std::lock_guard<std::mutex> lk(g_prof_mu);
  pa_status_t rc = PA_OK;
  for (const ProfEvent& pe : g_prof_pending) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(pe.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, pe.start, pe.stop);
    if (e != hipSuccess) rc = hip_fail(e, "profile event");
    if (pe.kind >= 0 && pe.kind < n) {
      ms[pe.kind] += t;
      launches[pe.kind] += 1;
    }
    g_prof_pool.push_back(pe.start);
    g_prof_pool.push_back(pe.stop);
  }
  g_prof_pending.clear();
  return rc;
}

}  // extern "C"
