// KV scatter: copy each new token's K and V rows into its paged-cache slot.
//
// Source: "[WebGPU] Initial PagedAttention implementation (1/n)", section
// "Description" (scatter of new K/V into the paged cache) and the review's
// check of the scatter block addressing.  With the cache laid out
// [num_blocks, block_size, num_kv_heads, head_size], slot s owns the
// contiguous row starting at element s * num_kv_heads * head_size, so the
// copy is row-to-row.  Each thread moves one 16-byte chunk of K and the
// matching chunk of V; a wavefront covers consecutive chunks of a row, so
// both the reads and the writes are fully coalesced 128-bit accesses.
#include "pa_common.hpp"
#include "pa_internal.hpp"

namespace pa {

__global__ __launch_bounds__(256) void scatter_kernel(const u32x4_t* __restrict__ k_new,
                                                      const u32x4_t* __restrict__ v_new,
                                                      const int32_t* __restrict__ slots,
                                                      u32x4_t* __restrict__ kc,
                                                      u32x4_t* __restrict__ vc,
                                                      int64_t total_chunks, int32_t row_chunks) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_chunks; i += stride) {
    const int64_t t = i / row_chunks;
    const int32_t c = (int32_t)(i - t * row_chunks);
    const int32_t s = slots[t];
    if (s < 0) continue;
    const int64_t dst = (int64_t)s * row_chunks + c;
    kc[dst] = k_new[i];
    vc[dst] = v_new[i];
  }
}

hipError_t launch_scatter(const void* k_new, const void* v_new, const int32_t* slots, void* kc,
                          void* vc, int64_t num_tokens, int32_t row_bytes, hipStream_t st) {
  const int32_t row_chunks = row_bytes / 16;
  const int64_t total = num_tokens * row_chunks;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     (const u32x4_t*)k_new, (const u32x4_t*)v_new, slots, (u32x4_t*)kc,
                     (u32x4_t*)vc, total, row_chunks);
  return hipGetLastError();
}

}  // namespace pa
