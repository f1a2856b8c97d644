// Host-side checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point's argument checks, the
// workspace-size arithmetic over a sweep of shapes up to the limits, and the
// full host path of pa_attention as far as the (stubbed) kernel launch.
// Prints one line per failed expectation and exits with their count.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pa.h"

static int g_failures = 0;
static void expect(pa_status_t got, pa_status_t want, const char* what) {
  if (got != want) {
    printf("FAIL %s: got %d (%s), want %d; last error: %s\n", what, (int)got,
           pa_status_string(got), (int)want, pa_last_error());
    ++g_failures;
  }
}

// Never dereferenced: every call below returns before a device access, or
// reaches a stubbed launch.
static void* const P = (void*)(uintptr_t)0x1000;
static const int32_t* const I = (const int32_t*)(uintptr_t)0x1000;
static const float* const F = (const float*)(uintptr_t)0x1000;
static void* const O = (void*)(uintptr_t)0x10000000;   // outputs, apart from every input range

int main() {
  // Status strings and the error buffer.
  if (strcmp(pa_status_string(PA_OK), "PA_OK") != 0) ++g_failures;
  if (strcmp(pa_status_string(12345), "PA_ERR_UNKNOWN") != 0) ++g_failures;

  // Workspace sizes: a sweep up to the limits; every size is either 0
  // (rejected shape) or 256-byte aligned and grows with num_tokens.
  const int32_t seqs[] = {1, 7, 256, 65536, 65537};
  const int64_t toks[] = {0, 1, 4096, 1 << 20, INT32_MAX, (int64_t)INT32_MAX + 1};
  const int32_t mbs[] = {1, 64, 16384, 16385};
  const int32_t heads[][2] = {{32, 8}, {64, 8}, {128, 1}, {4, 3}, {256, 1}};
  const int32_t dims[] = {64, 96, 128};
  const int32_t bss[] = {16, 24, 1024, 2048};
  for (int32_t b : seqs)
    for (int32_t mb : mbs)
      for (auto& h : heads)
        for (int32_t d : dims)
          for (int32_t bs : bss) {
            size_t prev = 0;
            for (int64_t t : toks) {
              const size_t n = pa_attention_workspace_size(b, t, mb, h[0], h[1], d, bs);
              if (n % 256 != 0) {
                printf("FAIL workspace %zu not 256-aligned\n", n);
                ++g_failures;
              }
              if (n != 0 && n < prev) {
                printf("FAIL workspace shrinks with num_tokens (%lld)\n", (long long)t);
                ++g_failures;
              }
              if (n != 0) prev = n;
            }
          }

  // pa_scatter_kv
  expect(pa_scatter_kv(P, P, I, P, P, 5, 8, 2, 60, 16, PA_F16, nullptr), PA_ERR_NOT_IMPLEMENTED,
         "scatter head_size 60");
  expect(pa_scatter_kv(P, P, I, P, P, -1, 8, 2, 64, 16, PA_F16, nullptr),
         PA_ERR_INVALID_ARGUMENT, "scatter negative tokens");
  expect(pa_scatter_kv(P, P, nullptr, P, P, 5, 8, 2, 64, 16, PA_F16, nullptr),
         PA_ERR_INVALID_ARGUMENT, "scatter null slots");
  expect(pa_scatter_kv(nullptr, nullptr, nullptr, P, P, 0, 8, 2, 64, 16, PA_F16, nullptr), PA_OK,
         "scatter empty");
  expect(pa_scatter_kv(P, P, I, P, P, 5, 8, 2, 64, 16, PA_BF16, nullptr), PA_ERR_HIP,
         "scatter valid (stubbed launch)");

  // pa_scatter_kv_paged / _fp8 / pa_seqlens_from_past
  expect(pa_scatter_kv_paged(P, P, I, I, I, P, P, 0, 5, 2, 8, 2, 64, 16, PA_F16, nullptr),
         PA_ERR_INVALID_ARGUMENT, "paged scatter no sequences");
  expect(pa_scatter_kv_paged(P, P, I, I, I, P, P, 2, 5, 1 << 28, 8, 2, 64, 16, PA_F16, nullptr),
         PA_ERR_NOT_IMPLEMENTED, "paged scatter table beyond INT32_MAX");
  expect(pa_scatter_kv_paged(P, P, I, I, I, P, P, 2, 5, 2, 8, 2, 64, 16, PA_F16, nullptr),
         PA_ERR_HIP, "paged scatter valid (stubbed launch)");
  expect(pa_scatter_kv_fp8(P, P, I, nullptr, F, P, P, 5, 8, 2, 64, 16, PA_F16, nullptr),
         PA_ERR_INVALID_ARGUMENT, "fp8 scatter null scale");
  expect(pa_scatter_kv_paged_fp8(P, P, I, I, I, F, nullptr, P, P, 2, 5, 2, 8, 2, 64, 16, PA_F16,
                                 nullptr),
         PA_ERR_INVALID_ARGUMENT, "fp8 paged scatter null scale");
  expect(pa_scatter_kv_paged_fp8(P, P, I, I, I, F, F, P, P, 2, 5, 1 << 28, 8, 2, 64, 16, PA_F16,
                                 nullptr),
         PA_ERR_NOT_IMPLEMENTED, "fp8 paged scatter table beyond INT32_MAX");
  expect(pa_scatter_kv_paged_fp8(P, P, I, I, I, F, F, P, P, 2, 5, 2, 8, 2, 64, 16, PA_BF16,
                                 nullptr),
         PA_ERR_HIP, "fp8 paged scatter valid (stubbed launch)");
  expect(pa_seqlens_from_past(I, nullptr, (int32_t*)P, 3, nullptr), PA_ERR_INVALID_ARGUMENT,
         "lengths null");

  // pa_rotary_scatter_kv
  expect(pa_rotary_scatter_kv(P, P, nullptr, P, P, 64, 64, 0, I, I, I, P, P, P, 2, 5, 2, 8, 4, 2,
                              64, 16, PA_F16, nullptr),
         PA_ERR_INVALID_ARGUMENT, "rotary key without value");
  expect(pa_rotary_scatter_kv(P, P, P, P, P, 64, 24, 0, I, I, I, P, P, P, 2, 5, 2, 8, 4, 2, 64, 16,
                              PA_F16, nullptr),
         PA_ERR_NOT_IMPLEMENTED, "rotary dim 24");
  expect(pa_rotary_scatter_kv(P, nullptr, nullptr, nullptr, nullptr, 0, 0, 0, I, I, I, P, P, P, 2,
                              5, 2, 8, 4, 2, 64, 16, PA_BF16, nullptr),
         PA_ERR_HIP, "rotary packed, no tables (stubbed launch)");

  // pa_attention: rejections, then the whole host path with a sized workspace.
  const size_t ws = pa_attention_workspace_size(2, 5, 2, 4, 2, 64, 16);
  expect(pa_attention(P, I, I, I, P, P, O, 2, 5, 2, 8, 0.125f, -1.f, 0, 4, 2, 64, 16, PA_F16, P,
                      ws, nullptr),
         PA_ERR_INVALID_ARGUMENT, "attention negative softcap");
  expect(pa_attention(P, I, I, I, P, P, O, 2, 5, 2, 8, 1e30f, 1e-40f, 0, 4, 2, 64, 16, PA_F16, P,
                      ws, nullptr),
         PA_ERR_INVALID_ARGUMENT, "attention scale/softcap overflow");
  expect(pa_attention(P, I, I, I, P, P, O, 2, 5, 2, 8, 0.125f, 0.f, 0, 4, 3, 64, 16, PA_F16, P,
                      ws, nullptr),
         PA_ERR_INVALID_ARGUMENT, "attention Hq % Hk");
  expect(pa_attention(P, I, I, I, P, P, O, 2, 5, 2, 8, 0.125f, 0.f, 0, 4, 2, 64, 16, PA_F16, P, 16,
                      nullptr),
         PA_ERR_WORKSPACE_TOO_SMALL, "attention small workspace");
  expect(pa_attention(P, I, I, I, P, P, O, 2, 5, 2, 8, 0.125f, 30.f, 128, 4, 2, 64, 16, PA_BF16,
                      P, ws, nullptr),
         PA_ERR_HIP, "attention valid (stubbed launch)");
  expect(pa_attention_fp8(P, I, I, I, P, P, F, F, O, 2, 5, 9, 2, 8, 0.125f, 0.f, 0, 4, 2, 64, 16,
                          PA_F16, P, ws, nullptr),
         PA_ERR_NOT_IMPLEMENTED, "fp8 attention q_len * G > 16");
  expect(pa_attention_fp8(P, I, I, I, P, P, F, F, O, 2, 5, 4, 2, 8, 0.125f, 0.f, 0, 4, 2, 64, 16,
                          PA_F16, P, ws, nullptr),
         PA_ERR_HIP, "fp8 attention valid (stubbed launch)");

  // pa_rotary_scatter_kv_fp8: the rotary step into fp8 caches.
  expect(pa_rotary_scatter_kv_fp8(P, P, P, P, P, 64, 64, 0, I, I, I, nullptr, F, O, P, P, 2, 5, 2,
                                  8, 4, 2, 64, 16, PA_F16, nullptr),
         PA_ERR_INVALID_ARGUMENT, "rotary fp8 null k_scale");
  expect(pa_rotary_scatter_kv_fp8(P, P, P, P, P, 64, 64, 1, I, I, I, F, F, O, P, P, 2, 5, 2, 8, 4,
                                  2, 64, 16, PA_BF16, nullptr),
         PA_ERR_HIP, "rotary fp8 valid (stubbed launch)");

  // pa_attention_rope: Q rows of the packed QKV stride, rotated on load.
  expect(pa_attention_rope(P, 4 * 64 - 8, P, P, 64, 64, 0, I, I, I, P, P, O, 2, 5, 2, 8, 0.125f,
                           0.f, 0, 4, 2, 64, 16, PA_F16, P, ws, nullptr),
         PA_ERR_INVALID_ARGUMENT, "rope attention row stride below Hq * D");
  expect(pa_attention_rope(P, 8 * 64, P, P, 64, 24, 0, I, I, I, P, P, O, 2, 5, 2, 8, 0.125f,
                           0.f, 0, 4, 2, 64, 16, PA_F16, P, ws, nullptr),
         PA_ERR_NOT_IMPLEMENTED, "rope attention rotary_dim 24");
  expect(pa_attention_rope(P, 8 * 64, P, P, 64, 64, 0, I, I, I, P, P, P, 2, 5, 2, 8, 0.125f,
                           0.f, 0, 4, 2, 64, 16, PA_F16, P, ws, nullptr),
         PA_ERR_INVALID_ARGUMENT, "rope attention out overlapping q");
  expect(pa_attention_rope(P, 8 * 64, P, P, 64, 64, 1, I, I, I, P, P, O, 2, 5, 2, 8, 0.125f,
                           0.f, 0, 4, 2, 64, 16, PA_BF16, P, ws, nullptr),
         PA_ERR_HIP, "rope attention valid (stubbed launch)");

  // pa_attention_rope_fp8: the rotated Q load over fp8 caches.
  expect(pa_attention_rope_fp8(P, 8 * 64, P, P, 64, 64, 0, I, I, I, P, P, F, F, O, 2, 5, 9, 2, 8,
                               0.125f, 0.f, 0, 4, 2, 64, 16, PA_F16, P, ws, nullptr),
         PA_ERR_NOT_IMPLEMENTED, "rope fp8 attention q_len * G > 16");
  expect(pa_attention_rope_fp8(P, 8 * 64, P, nullptr, 64, 64, 0, I, I, I, P, P, F, F, O, 2, 5, 4,
                               2, 8, 0.125f, 0.f, 0, 4, 2, 64, 16, PA_F16, P, ws, nullptr),
         PA_ERR_INVALID_ARGUMENT, "rope fp8 attention cos without sin");
  expect(pa_attention_rope_fp8(P, 8 * 64, P, P, 64, 64, 1, I, I, I, P, P, F, F, O, 2, 5, 4, 2, 8,
                               0.125f, 0.f, 0, 4, 2, 64, 16, PA_BF16, P, ws, nullptr),
         PA_ERR_HIP, "rope fp8 attention valid (stubbed launch)");

  // Shapes at the kernels' 32-bit limits, and misaligned tensors.
  if (pa_attention_workspace_size(1, 8, 1, 8191, 8191, 128, 1024) == 0) ++g_failures;
  if (pa_attention_workspace_size(1, 8, 1, 8192, 8192, 128, 1024) != 0) ++g_failures;
  if (pa_attention_workspace_size(65536, 65536, 16384, 64, 64, 128, 16) == 0) ++g_failures;
  if (pa_attention_workspace_size(65536, 65536, 16384, 65, 65, 128, 16) != 0) ++g_failures;
  expect(pa_attention(P, I, I, I, P, P, O, 65536, 5, 16384, 8, 0.125f, 0.f, 0, 65, 65, 128, 16,
                      PA_F16, P, ws, nullptr),
         PA_ERR_NOT_IMPLEMENTED, "attention decode items beyond 2^30");
  void* const P8 = (void*)(uintptr_t)0x1008;
  expect(pa_attention(P8, I, I, I, P, P, O, 2, 5, 2, 8, 0.125f, 0.f, 0, 4, 2, 64, 16, PA_F16, P,
                      ws, nullptr),
         PA_ERR_INVALID_ARGUMENT, "attention misaligned q");
  expect(pa_scatter_kv(P, P, I, P8, P, 5, 8, 2, 64, 16, PA_F16, nullptr),
         PA_ERR_INVALID_ARGUMENT, "scatter misaligned cache");

  // pa_attention_noalloc: rejections and the empty call return before any
  // HIP call (the scratch lookup needs a GPU).
  expect(pa_attention_noalloc(P, I, I, I, P, P, O, 256, 8432, 2048, 500224, 0.088f, 0.f, 0, 64, 8,
                              128, 16, PA_BF16, nullptr),
         PA_ERR_WORKSPACE_TOO_SMALL, "noalloc workspace beyond the fixed scratch");
  expect(pa_attention_noalloc(P, I, I, I, P, P, O, 2, 5, 2, 8, 0.125f, 0.f, 0, 4, 3, 64, 16,
                              PA_F16, nullptr),
         PA_ERR_INVALID_ARGUMENT, "noalloc Hq % Hk");
  expect(pa_attention_noalloc(nullptr, I, I, I, P, P, nullptr, 2, 0, 2, 8, 0.125f, 0.f, 0, 4, 2,
                              64, 16, PA_F16, nullptr),
         PA_OK, "noalloc empty call");

  // Metadata validator and profiling arguments.
  uint32_t viol = 0;
  expect(pa_validate_metadata(nullptr, I, I, nullptr, 2, 5, 2, 8, 16, &viol, nullptr),
         PA_ERR_INVALID_ARGUMENT, "validator null cu");
  expect(pa_profile_read(nullptr, nullptr, 4), PA_ERR_INVALID_ARGUMENT, "profile null arrays");

  printf("%d failure(s)\n", g_failures);
  return g_failures;
}
