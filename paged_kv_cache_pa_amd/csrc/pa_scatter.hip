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
    kc[dst] = __builtin_nontemporal_load(&k_new[i]);   // new rows are read once
    vc[dst] = __builtin_nontemporal_load(&v_new[i]);
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

// Scatter into fp8 (e4m3) caches with per-channel scales: the quantized KV
// cache ("[WebGPU] Initial PagedAttention implementation (1/n)", "Roadmap",
// phase 3: a cache element type apart from the query type, quantized KV
// first).  The pages define no format; the one taken: OCP e4m3 elements and
// one float32 scale per (KV head, channel) for K and for V.  Element x of a
// row is stored as e4m3(y), y = x * (1 / scale) with the reciprocal and the
// product rounded to fp32, |y| > 448 (infinities too) saturated to 448, NaN
// kept, then rounded to nearest even by v_cvt_pk_fp8_f32 (which alone would
// turn magnitudes above 464 into NaN).  Each thread quantizes one chunk of
// 8 elements: a 16-byte load of K and of V, two 16-byte scale loads each, and
// an 8-byte store of codes per cache (quantize8, shared with the rotary
// scatter into fp8 caches).
template <typename T>
__global__ __launch_bounds__(256) void scatter_fp8_kernel(
    const u32x4_t* __restrict__ k_new, const u32x4_t* __restrict__ v_new,
    const int32_t* __restrict__ slots, const float4_t* __restrict__ k_scale,
    const float4_t* __restrict__ v_scale, u32x2_t* __restrict__ kc, u32x2_t* __restrict__ vc,
    int64_t total_chunks, int32_t row_chunks) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_chunks; i += stride) {
    const int64_t t = i / row_chunks;
    const int32_t c = (int32_t)(i - t * row_chunks);
    const int32_t s = slots[t];
    if (s < 0) continue;
    const int64_t dst = (int64_t)s * row_chunks + c;
    const u32x4_t kx = __builtin_nontemporal_load(&k_new[i]);   // new rows are read once
    const u32x4_t vx = __builtin_nontemporal_load(&v_new[i]);
    kc[dst] = quantize8<T>(kx, k_scale[2 * c], k_scale[2 * c + 1]);
    vc[dst] = quantize8<T>(vx, v_scale[2 * c], v_scale[2 * c + 1]);
  }
}

hipError_t launch_scatter_fp8(const void* k_new, const void* v_new, const int32_t* slots,
                              const float* k_scale, const float* v_scale, void* kc, void* vc,
                              int64_t num_tokens, int32_t row_elems, int32_t dtype,
                              hipStream_t st) {
  const int32_t row_chunks = row_elems / 8;
  const int64_t total = num_tokens * row_chunks;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  auto kern = dtype == 1 ? scatter_fp8_kernel<BF16> : scatter_fp8_kernel<F16>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, st, (const u32x4_t*)k_new,
                     (const u32x4_t*)v_new, slots, (const float4_t*)k_scale,
                     (const float4_t*)v_scale, (u32x2_t*)kc, (u32x2_t*)vc, total, row_chunks);
  return hipGetLastError();
}

// Scatter with the slots computed on the device from the batch metadata
// ("[WebGPU] Initial PagedAttention implementation (1/n)", section
// "Description": the op derives each new token's cache slot from the
// cumulative query lengths, the past lengths and the block table; the
// review's checks of the token-to-sequence scan and the scatter block
// addressing).  One wavefront per new token t: the first sequence b with
// cu[b+1] > t (binary search, wave-uniform), KV position
// pos = past_b + (t - cu[b]) with past_b = seqlens_kv[b] - q_len_b, slot =
// block_table[b][pos / bs] * bs + pos % bs; then the row copy as above.  A
// negative table entry skips the token.
// KV8: the caches hold e4m3 codes; each 8-element chunk is quantized as in
// scatter_fp8_kernel (quantize8, per-channel scales) instead of copied, so
// the codes equal those of pa_scatter_kv_fp8 on the same slots.
template <typename T, bool KV8>
__global__ __launch_bounds__(256) void scatter_paged_kernel(
    const u32x4_t* __restrict__ k_new, const u32x4_t* __restrict__ v_new,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ table, void* __restrict__ kc, void* __restrict__ vc,
    const float4_t* __restrict__ k_scale, const float4_t* __restrict__ v_scale,
    int32_t num_seqs, int64_t num_tokens, int32_t max_blocks, int32_t block_size,
    int32_t row_chunks) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); t < num_tokens;
       t += nwaves) {
    // first b in [0, num_seqs) with cu[b + 1] > t
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(cu[mid + 1]) > t) hi = mid; else lo = mid + 1;
    }
    const int b = lo;
    const int c0 = __builtin_amdgcn_readfirstlane(cu[b]);
    const int q_len = __builtin_amdgcn_readfirstlane(cu[b + 1]) - c0;
    const int past = __builtin_amdgcn_readfirstlane(lens[b]) - q_len;
    const int pos = past + (int)(t - c0);
    const int blk = __builtin_amdgcn_readfirstlane(table[(int64_t)b * max_blocks + pos / block_size]);
    if (blk < 0) continue;
    const int64_t slot = (int64_t)blk * block_size + pos % block_size;
    for (int c = lane; c < row_chunks; c += 64) {
      const int64_t src = t * row_chunks + c;
      const int64_t dst = slot * row_chunks + c;
      const u32x4_t kx = __builtin_nontemporal_load(&k_new[src]);   // new rows are read once
      const u32x4_t vx = __builtin_nontemporal_load(&v_new[src]);
      if constexpr (KV8) {
        reinterpret_cast<u32x2_t*>(kc)[dst] = quantize8<T>(kx, k_scale[2 * c], k_scale[2 * c + 1]);
        reinterpret_cast<u32x2_t*>(vc)[dst] = quantize8<T>(vx, v_scale[2 * c], v_scale[2 * c + 1]);
      } else {
        reinterpret_cast<u32x4_t*>(kc)[dst] = kx;
        reinterpret_cast<u32x4_t*>(vc)[dst] = vx;
      }
    }
  }
}

hipError_t launch_scatter_paged(const void* k_new, const void* v_new, const int32_t* cu,
                                const int32_t* lens, const int32_t* table, void* kc, void* vc,
                                const float* k_scale, const float* v_scale, int32_t num_seqs,
                                int64_t num_tokens, int32_t max_blocks, int32_t block_size,
                                int32_t row_elems, int32_t dtype, bool kv8, hipStream_t st) {
  int64_t blocks = (num_tokens + 3) / 4;   // 4 waves (tokens) per work-group
  if (blocks > 16384) blocks = 16384;
  // 16-bit caches: a byte copy, the same kernel for both dtypes.
  auto kern = !kv8 ? scatter_paged_kernel<F16, false>
              : dtype == 1 ? scatter_paged_kernel<BF16, true> : scatter_paged_kernel<F16, true>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, st, (const u32x4_t*)k_new,
                     (const u32x4_t*)v_new, cu, lens, table, kc, vc, (const float4_t*)k_scale,
                     (const float4_t*)v_scale, num_seqs, num_tokens, max_blocks, block_size,
                     row_elems / 8);
  return hipGetLastError();
}

// seqlens_kv[b] = past_seqlens[b] + q_len_b: total KV lengths from the past
// lengths the pages' op takes ("FlashAttention: optional seqlens_q input").
__global__ __launch_bounds__(256) void seqlens_from_past_kernel(const int32_t* __restrict__ cu,
                                                                const int32_t* __restrict__ past,
                                                                int32_t* __restrict__ out,
                                                                int32_t num_seqs) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < num_seqs) out[b] = past[b] + (cu[b + 1] - cu[b]);
}

hipError_t launch_seqlens_from_past(const int32_t* cu, const int32_t* past, int32_t* out,
                                    int32_t num_seqs, hipStream_t st) {
  hipLaunchKernelGGL(seqlens_from_past_kernel, dim3((unsigned)((num_seqs + 255) / 256)), dim3(256),
                     0, st, cu, past, out, num_seqs);
  return hipGetLastError();
}

}  // namespace pa
