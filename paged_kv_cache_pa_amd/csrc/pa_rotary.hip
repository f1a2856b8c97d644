// The steps ahead of the attention for one batch of new tokens, in one pass:
// split packed QKV rows, rotate Q and K by the rotary position embedding at
// each token's KV position, write the rotated Q for the attention and the
// rotated K and plain V into the paged caches (16-bit, or fp8 with
// per-channel scales; without a Q output, the Q rows are skipped:
// pa_attention_rope rotates Q as it loads it).
//
// Sources: "[WebGPU] Initial PagedAttention implementation (1/n)", the file
// summaries (a packed-QKV split program and a rotary program ahead of the
// scatter) and the review's summary (interleaved and split pairing, the
// sign of the rotation, pass-through of dimensions from rotary_dim on); the
// rotation is the rotary position embedding of Su et al. (RoFormer),
// section 3.2.  The pages run these as separate programs with a round trip
// through memory each; here the split, both rotations and the scatter are
// one kernel that reads every new element once and writes it once.
//
// One wavefront per token.  The token's rows (num_heads Q rows, num_kv_heads
// K rows, num_kv_heads V rows) are cut into 16-byte chunks of 8 elements;
// the wave's lanes take consecutive chunks, so reads and writes are
// coalesced.  rotary_dim is a multiple of 16, so a chunk never straddles
// the rotary boundary or the half of a split pair: with interleaved pairing
// a chunk holds 4 whole pairs; with split pairing a chunk in the first half
// is completed by the chunk rotary_dim / 2 elements on (and vice versa),
// which the lane loads itself.  Arithmetic in fp32, one rounding (to
// nearest even) into the element type.
#include "pa_common.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {

__device__ inline u32x4_t ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }
// The new Q/K/V rows are read once (a chunk and its split-pairing partner
// are each read twice, by neighbouring lanes of one wave): non-temporal
// loads, measured 20 % faster than cached ones.
__device__ inline u32x4_t ld16_once(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ inline u32x2_t ld8(const uint16_t* p) { return *reinterpret_cast<const u32x2_t*>(p); }

}  // namespace

// KV8: fp8 (e4m3) caches with per-channel scales: each K chunk, rotated and
// rounded to T as for 16-bit caches, and each V chunk are quantized by the
// fp8 scatter's quantize8, so the codes are those pa_scatter_kv_fp8 writes
// for the rotated rows.
template <typename T, bool ROT, bool INTER, bool KV8>
__global__ __launch_bounds__(256) void rotary_scatter_kernel(RotaryArgs a) {
  const int lane = threadIdx.x & 63;
  const int hq = a.num_heads, hk = a.num_kv_heads, hd = a.head_size;
  const int cpr = hd >> 3;                       // chunks per head row
  const int nrows = hq + 2 * hk;
  const int nchunks = nrows * cpr;
  const int half = a.rotary_dim >> 1;
  const uint16_t* __restrict__ qsrc = (const uint16_t*)a.query;
  const uint16_t* __restrict__ ksrc = (const uint16_t*)a.key;
  const uint16_t* __restrict__ vsrc = (const uint16_t*)a.value;
  const uint16_t* __restrict__ cosp = (const uint16_t*)a.cos_cache;
  const uint16_t* __restrict__ sinp = (const uint16_t*)a.sin_cache;
  uint16_t* __restrict__ qo = (uint16_t*)a.q_out;
  const bool packed = ksrc == nullptr;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
       t < a.num_tokens; t += nwaves) {
    // Sequence of token t: the first b with cu[b + 1] > t (wave-uniform).
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(a.cu[mid + 1]) > t) hi = mid; else lo = mid + 1;
    }
    const int b = lo;
    const int c0 = __builtin_amdgcn_readfirstlane(a.cu[b]);
    const int q_len = __builtin_amdgcn_readfirstlane(a.cu[b + 1]) - c0;
    const int pos = __builtin_amdgcn_readfirstlane(a.lens[b]) - q_len + (int)(t - c0);
    // Preconditions (lengths >= q_len; positions inside the tables): a token
    // that breaks them is skipped whole.
    if (pos < 0 || (ROT && pos >= a.max_position)) continue;
    const int bi = pos / a.block_size;
    const int blk = bi < a.max_blocks
        ? __builtin_amdgcn_readfirstlane(a.table[(int64_t)b * a.max_blocks + bi]) : -1;
    const bool write_kv = blk >= 0;   // a negative table entry: no cache slot
    const int64_t slot = (int64_t)blk * a.block_size + pos % a.block_size;
    const uint16_t* crow = cosp + (int64_t)pos * half;
    const uint16_t* srow = sinp + (int64_t)pos * half;

    // Without q_out the Q rows are left to the attention's rotated Q load.
    for (int c = lane + (qo == nullptr ? hq * cpr : 0); c < nchunks; c += 64) {
      const int r = c / cpr;                      // row: Q heads, K heads, V heads
      const int e = (c - r * cpr) * 8;            // first element of the chunk
      const uint16_t* src;
      uint16_t* dst = nullptr;   // a Q row
      void* cache = nullptr;     // or element cel of a cache
      int64_t cel = 0;
      const float* scale = nullptr;
      if (r < hq) {
        src = packed ? qsrc + (t * nrows + r) * hd : qsrc + (t * hq + r) * hd;
        dst = qo + (t * hq + r) * hd;
      } else if (r < hq + hk) {
        if (!write_kv) continue;
        src = packed ? qsrc + (t * nrows + r) * hd : ksrc + (t * hk + r - hq) * hd;
        cache = a.k_cache;
        cel = (slot * hk + r - hq) * hd;
        scale = a.k_scale + (int64_t)(r - hq) * hd;
      } else {
        if (!write_kv) continue;
        src = packed ? qsrc + (t * nrows + r) * hd : vsrc + (t * hk + r - hq - hk) * hd;
        cache = a.v_cache;
        cel = (slot * hk + r - hq - hk) * hd;
        scale = a.v_scale + (int64_t)(r - hq - hk) * hd;
      }
      u32x4_t x = ld16_once(src + e);
      if (ROT && r < hq + hk && e < a.rotary_dim) {
        if constexpr (INTER) {
          x = rope_interleaved<T>(x, ld8(crow + e / 2), ld8(srow + e / 2));
        } else {
          const bool first = e < half;
          const int k = first ? e : e - half;      // pair index of the chunk's first element
          const u32x4_t y = ld16_once(src + (first ? e + half : e - half));
          x = rope_split<T>(x, y, ld16(crow + k), ld16(srow + k), first);
        }
      }
      if (r < hq) {
        *reinterpret_cast<u32x4_t*>(dst + e) = x;
      } else if constexpr (KV8) {
        const float4_t* sc = reinterpret_cast<const float4_t*>(scale + e);
        *reinterpret_cast<u32x2_t*>((uint8_t*)cache + cel + e) = quantize8<T>(x, sc[0], sc[1]);
      } else {
        *reinterpret_cast<u32x4_t*>((uint16_t*)cache + cel + e) = x;
      }
    }
  }
}

template <typename T, bool KV8>
static void rotary_dispatch(const RotaryArgs& a, dim3 g, hipStream_t st) {
  const dim3 blk(256);
  if (a.cos_cache == nullptr)
    hipLaunchKernelGGL((rotary_scatter_kernel<T, false, false, KV8>), g, blk, 0, st, a);
  else if (a.interleaved)
    hipLaunchKernelGGL((rotary_scatter_kernel<T, true, true, KV8>), g, blk, 0, st, a);
  else
    hipLaunchKernelGGL((rotary_scatter_kernel<T, true, false, KV8>), g, blk, 0, st, a);
}

hipError_t launch_rotary_scatter(const RotaryArgs& a, int dtype, hipStream_t st) {
  int64_t blocks = (a.num_tokens + 3) / 4;   // 4 waves (tokens) per work-group
  if (blocks > 16384) blocks = 16384;
  const dim3 g((unsigned)blocks);
  const bool kv8 = a.k_scale != nullptr;
  if (dtype == 0)
    kv8 ? rotary_dispatch<F16, true>(a, g, st) : rotary_dispatch<F16, false>(a, g, st);
  else
    kv8 ? rotary_dispatch<BF16, true>(a, g, st) : rotary_dispatch<BF16, false>(a, g, st);
  return hipGetLastError();
}

}  // namespace pa
