// The attention kernel: one persistent launch that runs both kinds of work
// item the plan produced, prefill tiles (matrix-core bound) and split-KV
// decode items (HBM bound), plus the split-KV combine.
//
// Sources: "[WebGPU] Initial PagedAttention implementation (1/n)" -
// "Description" (one attention pass over a continuous batch that mixes
// prefill chunks and decode tokens) and "Roadmap" (phase 2: page-aware
// prefill and decode kernels reading K/V through the block table).
//
// Run back to back, the two kinds of work leave one MI355X resource idle in
// turn: prefill keeps the matrix cores busy while HBM idles, decode streams
// HBM while the matrix cores idle, and one CU streams only ~40 GB/s, so
// decode needs many CUs for full bandwidth.  Here each work-group (8 waves,
// one per CU) takes a role at start: the first counters[kPrefillFirst]
// groups (spread over the XCDs by the round-robin dispatch) run prefill
// items and the rest run decode items, both at once; a group whose queue
// runs dry moves to the other kind, so the tail balances itself.  The plan
// kernel sizes the split so that both halves finish together under the cost
// model kPrefillStepCost.
#include "pa_decode.hpp"
#include "pa_prefill.hpp"

namespace pa {

// CAP / WIN: the score soft cap / the sliding window is on (separate
// instantiations, so the plain kernel carries no code for either).
template <typename T, int D, bool CAP, bool WIN>
__global__ __launch_bounds__(512, 1) void attention_kernel(AttnArgs a) {
  const bool prefill_first = (int)blockIdx.x < a.counters[kPrefillFirst];
  // Straight-line phases (no loop around them, so nothing of one body is
  // hoisted to stay live across the other); the small decode body appears
  // twice, the large prefill body once.
  if (!prefill_first) decode_items<T, D, false, CAP, WIN>(a);
  prefill_items<T, D, CAP, WIN>(a);
  if (prefill_first) decode_items<T, D, false, CAP, WIN>(a);
}

// fp8 caches: decode items only (the plan gives every sequence the decode
// path); waves are independent and use no LDS.
template <typename T, int D, bool CAP, bool WIN>
__global__ __launch_bounds__(512) void attention_kernel_fp8(AttnArgs a) {
  decode_items<T, D, true, CAP, WIN>(a);
}

template <typename T, int D>
static const void* attention_fn(bool kv8) {
  return kv8 ? (const void*)&attention_kernel_fp8<T, D, false, false>
             : (const void*)&attention_kernel<T, D, false, false>;
}

static const void* attention_fn(int dtype, int head_size, bool kv8) {
  if (dtype == 0)
    return head_size == 128 ? attention_fn<F16, 128>(kv8) : attention_fn<F16, 64>(kv8);
  return head_size == 128 ? attention_fn<BF16, 128>(kv8) : attention_fn<BF16, 64>(kv8);
}

// One work-group per CU whatever the variant (launch bounds 512, 1), so the
// uncapped kernel sizes the grid for all of them.
int attention_workers(int dtype, int head_size, int num_cus, bool kv8) {
  return resident_blocks(attention_fn(dtype, head_size, kv8), num_cus, 512);
}

template <typename T, int D>
static void attention_launch(const AttnArgs& a, dim3 g, hipStream_t st, bool kv8) {
  const dim3 b(512);
  const bool cap = a.cap_b > 0.f, win = a.window > 0;
  if (kv8 && cap && win)
    hipLaunchKernelGGL((attention_kernel_fp8<T, D, true, true>), g, b, 0, st, a);
  else if (kv8 && cap)
    hipLaunchKernelGGL((attention_kernel_fp8<T, D, true, false>), g, b, 0, st, a);
  else if (kv8 && win)
    hipLaunchKernelGGL((attention_kernel_fp8<T, D, false, true>), g, b, 0, st, a);
  else if (kv8)
    hipLaunchKernelGGL((attention_kernel_fp8<T, D, false, false>), g, b, 0, st, a);
  else if (cap && win)
    hipLaunchKernelGGL((attention_kernel<T, D, true, true>), g, b, 0, st, a);
  else if (cap)
    hipLaunchKernelGGL((attention_kernel<T, D, true, false>), g, b, 0, st, a);
  else if (win)
    hipLaunchKernelGGL((attention_kernel<T, D, false, true>), g, b, 0, st, a);
  else
    hipLaunchKernelGGL((attention_kernel<T, D, false, false>), g, b, 0, st, a);
}

template <typename T>
static hipError_t attention_dispatch(const AttnArgs& a, int head_size, int grid, hipStream_t st,
                                     bool kv8) {
  const dim3 g((unsigned)grid);
  if (head_size == 128)
    attention_launch<T, 128>(a, g, st, kv8);
  else
    attention_launch<T, 64>(a, g, st, kv8);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int dtype, int head_size, int grid,
                            hipStream_t st, bool kv8) {
  return dtype == 0 ? attention_dispatch<F16>(a, head_size, grid, st, kv8)
                    : attention_dispatch<BF16>(a, head_size, grid, st, kv8);
}

template <typename T>
static hipError_t combine_dispatch(const AttnArgs& a, int head_size, hipStream_t st) {
  dim3 grid(a.num_seqs, a.num_kv_heads);
  if (head_size == 128)
    hipLaunchKernelGGL((combine_kernel<T, 128>), grid, dim3(kCombineThreads), 0, st, a);
  else
    hipLaunchKernelGGL((combine_kernel<T, 64>), grid, dim3(kCombineThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_combine(const AttnArgs& a, int dtype, int head_size, hipStream_t st) {
  return dtype == 0 ? combine_dispatch<F16>(a, head_size, st)
                    : combine_dispatch<BF16>(a, head_size, st);
}

}  // namespace pa
