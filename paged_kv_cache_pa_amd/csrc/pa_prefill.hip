// Prefill path: causal paged attention for sequences with more than one
// 16-column tile of (token, head-in-group) query rows, on the matrix cores.
//
// Sources: "[WebGPU] Initial PagedAttention implementation (1/n)" -
// "FlashAttention: optional seqlens_q input" (row i of sequence b sees keys
// 0..past_b+i with past_b = total_kv_b - q_len_b; the causal length is
// past + i + 1) and "Roadmap" (phase 2: page-aware prefill kernels that read
// K/V straight from the paged cache); FlexAttention operator page -
// "FlexAttention Computation" and "Grouped Query Attention (GQA)".
//
// Work item = (sequence b, KV head kh, tile): 128 query rows, row r being
// token i0 + r / G of the tile and query head kh*G + r % G, so the G heads
// that share kh share every K/V tile.  Items come from 8 per-XCD queues
// (work-group w serves queue w % 8 first, then steals from the others).
// Each of the 4 waves owns 32 rows (two 16-row groups).  Per 64-key tile:
//   K, V rows resolved through the block table (one block id per wave per
//   tile), copied HBM -> LDS by 128-bit direct-to-LDS loads, double buffered
//   S^T = K . Q^T          16x16x32 MFMA (fp16/bf16 in, fp32 acc)
//   causal mask key <= past + i, online softmax in fp32 (exp2)
//   O^T += V^T . P^T       16x16x32 MFMA, P rounded to the input dtype
// Key tiles beyond the tile's last visible key are never loaded, and a wave
// skips the matrix work of key tiles that lie wholly above its rows'
// diagonal; the causal mask is applied only on tiles that cross a row's
// diagonal, and the output accumulators are rescaled only when a row's
// running max moves.  Key rows past the visible range are replaced by the
// last visible row, so NaN in unused cache slots never enters LDS.
#include "pa_common.hpp"
#include "pa_internal.hpp"

namespace pa {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) short4_t* lds_s4_t;

// xor-16 / xor-32 lane exchanges as VALU permutes (no LDS round trip).
__device__ inline float max_xor16_32(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float sum_xor16_32(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// K/V tiles live in LDS as unpadded rows of D halfs whose 16-byte chunks are
// XOR-swizzled by the row index (chunk c of row r sits in slot
// c ^ (r % (D/8))), which keeps both the row-wise K reads and the
// column-wise V reads free of bank conflicts.  The tiles are filled by
// global_load_lds_dwordx4 (HBM/L2 -> LDS without registers), double
// buffered: the loads of tile i+1 are in flight while tile i is computed.
template <typename T, int D>
__global__ __launch_bounds__(256, 2) void prefill_kernel(AttnArgs a) {
  constexpr int NS = D / 32;            // QK^T steps
  constexpr int NT = D / 16;            // O^T tiles (halfs per lane per V row)
  constexpr int BN = kPrefillKeys;      // keys per K/V tile
  constexpr int ROWB = D * 2;           // bytes per K/V row
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int RPI = 1024 / ROWB;      // rows per wave-wide 1 KiB LDS load
  constexpr int LPW = 16 / RPI;         // loads per wave per operand (16 rows)
  constexpr int TB = BN * ROWB;         // bytes per operand tile
  // Two separate LDS objects (not one array indexed by buffer) so the
  // compiler can tell the prefetch target from the tile being read and does
  // not wait for the prefetch before reading.
  __shared__ __attribute__((aligned(1024))) unsigned char lds0[2 * TB];   // [K, V]
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[2 * TB];
  __shared__ int item_sh;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int hk = a.num_kv_heads, G = a.group, hq = a.num_heads;
  const int TQ = a.tokens_per_tile;
  const int bsz = a.block_size, shift = a.block_shift;
  const int64_t row_stride = (int64_t)hk * D;
  const float c = a.scale_log2;
  const uint16_t* __restrict__ qp = (const uint16_t*)a.q;
  const uint16_t* __restrict__ kc = (const uint16_t*)a.k_cache;
  const uint16_t* __restrict__ vc = (const uint16_t*)a.v_cache;
  uint16_t* __restrict__ op = (uint16_t*)a.out;
  const int home = blockIdx.x % kQueues;

  // Slot of 16-byte chunk `chunk` of tile row `row`: XOR with the row's low
  // log2(CPR) bits rotated left by one.  Row-wise K reads (16 rows, one
  // chunk) and transposed V reads (4 rows, two adjacent chunks) then touch
  // distinct slots.
  constexpr int CB = CPR == 16 ? 4 : 3;
  auto swz = [](int row) { return ((row << 1) | ((row >> (CB - 1)) & 1)) & (CPR - 1); };
  auto slot = [&](int row, int chunk) { return row * ROWB + ((chunk ^ swz(row)) << 4); };

  for (int qi = 0; qi < kQueues; ++qi) {
    const int x = (home + qi) % kQueues;
    const int qlen = a.counters[kQueueLen + x];
    const int qstart = a.counters[kQueueStart + x];
    for (;;) {
      if (tid == 0) item_sh = atomicAdd(a.counters_rw + kCtrPrefill + x, 1);
      __syncthreads();
      const int k = __builtin_amdgcn_readfirstlane(item_sh);   // uniform: scalar loads below
      __syncthreads();
      if (k >= qlen) break;
      const int4 itm = a.pf_items[qstart + k];
      const int b = itm.x, kh = itm.y, tile = itm.z;
      const SeqInfo si = a.seqinfo[b];
      const int ql = si.q_len, L = si.kv_len;
      const int past = L - ql;
      const int i0 = tile * TQ;
      const int last_tok = min(i0 + TQ, ql) - 1;
      const int kend = past + last_tok + 1;   // keys visible to the tile's last row
      const int32_t* trow = a.block_table + (int64_t)b * a.max_blocks_per_seq;

      // Rows [16*wave, 16*wave+16) of the K and V tiles starting at key kt;
      // keys at or past kend are clamped onto key kend-1 (finite data, masked).
      // Block id of this wave's 16-row group of the tile at key kt (one
      // scalar load; rows of a group never straddle a block).
      auto block_of = [&](int kt) { return trow[min(kt + 16 * wave, kend - 1) >> shift]; };
      auto issue = [&](int kt, unsigned char* dst, int blk) {
        const int64_t blk_row = (int64_t)blk * bsz;
        unsigned char* kdst = dst + 16 * wave * ROWB;
#pragma unroll
        for (int p = 0; p < LPW; ++p) {
          const int row = 16 * wave + p * RPI + lane / CPR;
          const int j = min(kt + row, kend - 1);
          const int gch = (lane % CPR) ^ swz(row);
          const int64_t off = (blk_row + (j & (bsz - 1))) * row_stride + (int64_t)kh * D + gch * 8;
          __builtin_amdgcn_global_load_lds(kc + off, (lds_ptr_t)(kdst + p * 1024), 16, 0, 0);
          __builtin_amdgcn_global_load_lds(vc + off, (lds_ptr_t)(kdst + TB + p * 1024), 16, 0, 0);
        }
      };
      issue(0, lds0, block_of(0));
      int blk_next = BN < kend ? block_of(BN) : 0;   // fetched one tile ahead

      // Q^T operands and causal limits of this lane's two row groups.
      u32x4_t qreg[2][NS];
      int limit[2], tok[2], head[2];
#pragma unroll
      for (int rho = 0; rho < 2; ++rho) {
        const int row = 32 * wave + 16 * rho + r16;
        const int ti = i0 + row / G;
        const bool valid = row < TQ * G && ti < ql;
        tok[rho] = valid ? si.cu + ti : -1;
        head[rho] = kh * G + row % G;
        limit[rho] = valid ? past + ti : -1;
        const uint16_t* qrow = qp + ((int64_t)(valid ? tok[rho] : 0) * hq + head[rho]) * D;
#pragma unroll
        for (int s = 0; s < NS; ++s)
          qreg[rho][s] = valid ? ld16(qrow + (4 * s + kq) * 8) : u32x4_t{0, 0, 0, 0};
      }
      int wave_kmax = max(limit[0], limit[1]);
      int wave_kmin = min(limit[0], limit[1]);
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        wave_kmax = max(wave_kmax, __shfl_xor(wave_kmax, o));
        wave_kmin = min(wave_kmin, __shfl_xor(wave_kmin, o));
      }

      float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
      float4_t acc[2][NT];
#pragma unroll
      for (int rho = 0; rho < 2; ++rho)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[rho][t] = float4_t{0.f, 0.f, 0.f, 0.f};

      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      auto step = [&](int kt, const unsigned char* cur, unsigned char* nxt) {
        if (kt + BN < kend) {
          issue(kt + BN, nxt, blk_next);
          blk_next = kt + 2 * BN < kend ? block_of(kt + 2 * BN) : 0;
        }
        const unsigned char* kb = cur;
        const unsigned char* vb = cur + TB;

        if (kt <= wave_kmax) {   // else: tile wholly above this wave's diagonal
          float4_t sacc[4][2];
#pragma unroll
          for (int kap = 0; kap < 4; ++kap) {
            sacc[kap][0] = float4_t{0.f, 0.f, 0.f, 0.f};
            sacc[kap][1] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(kb + slot(16 * kap + r16, 4 * s + kq));
              sacc[kap][0] = Elt<T>::mfma32(ka, qreg[0][s], sacc[kap][0]);
              sacc[kap][1] = Elt<T>::mfma32(ka, qreg[1][s], sacc[kap][1]);
            }
          }

          const bool diag = kt + BN - 1 > wave_kmin;   // some row needs the causal mask here
          u32x4_t pb[2][2];
#pragma unroll
          for (int rho = 0; rho < 2; ++rho) {
            float sv[4][4];
            float mt = -INFINITY;
            if (diag) {
#pragma unroll
              for (int kap = 0; kap < 4; ++kap)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int key = kt + 16 * kap + 4 * kq + i;
                  sv[kap][i] = key <= limit[rho] ? sacc[kap][rho][i] * c : -INFINITY;
                  mt = fmaxf(mt, sv[kap][i]);
                }
            } else {
              float hi = -INFINITY, lo = INFINITY;
#pragma unroll
              for (int kap = 0; kap < 4; ++kap)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  hi = fmaxf(hi, sacc[kap][rho][i]);
                  lo = fminf(lo, sacc[kap][rho][i]);
                }
              mt = c >= 0.f ? hi * c : lo * c;
            }
            mt = max_xor16_32(mt);
            const float m_new = fmaxf(m[rho], mt);
            const float base_m = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = exp2_fast(m[rho] - base_m);
            if (diag) {
#pragma unroll
              for (int kap = 0; kap < 4; ++kap)
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[kap][i] = exp2_fast(sv[kap][i] - base_m);
            } else {
#pragma unroll
              for (int kap = 0; kap < 4; ++kap)
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[kap][i] = exp2_fast(fmaf(sacc[kap][rho][i], c, -base_m));
            }
            if (__any(alpha != 1.f)) {   // rescale only when some row's max moved
#pragma unroll
              for (int t = 0; t < NT; ++t) acc[rho][t] *= alpha;
            }
            // P rounded to the input dtype feeds P.V; the denominator sums
            // the same rounded values.
            float psum = 0.f;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              pb[rho][u] = u32x4_t{Elt<T>::pack2(sv[2 * u][0], sv[2 * u][1]),
                                   Elt<T>::pack2(sv[2 * u][2], sv[2 * u][3]),
                                   Elt<T>::pack2(sv[2 * u + 1][0], sv[2 * u + 1][1]),
                                   Elt<T>::pack2(sv[2 * u + 1][2], sv[2 * u + 1][3])};
#pragma unroll
              for (int w = 0; w < 4; ++w) psum = Elt<T>::sum2(pb[rho][u][w], psum);
            }
            l[rho] = l[rho] * alpha + psum;
            m[rho] = m_new;
          }

          // O^T tile t covers d = 16t .. 16t+15.  ds_read_b64_tr_b16: within
          // each 16-lane group, result lane i gets element i % 4 of the
          // 8 bytes read by source lanes 4r + i / 4 (r = 0..3).  Source lane
          // (kq, r, q) reads key row 4kq + r at d = 16t + 4q .. +3, so lane i
          // receives d = 16t + i of keys 4kq .. 4kq+3: the V^T operand, with
          // contraction element e <-> key 32u + 4kq + e (e < 4) or
          // 32u + 16 + 4kq + (e - 4), the same keys pb holds.
          const int r4 = (lane & 15) >> 2, q4 = lane & 3;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int R0 = 32 * u + 4 * kq + r4;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              const int chunk = 2 * t + (q4 >> 1);
              const int boff = (q4 & 1) << 3;
              const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_s4_t)(vb + slot(R0, chunk) + boff));
              const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_s4_t)(vb + slot(R0 + 16, chunk) + boff));
              const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo);
              const u32x2_t h2 = __builtin_bit_cast(u32x2_t, hi);
              const u32x4_t va = {l2[0], l2[1], h2[0], h2[1]};
              acc[0][t] = Elt<T>::mfma32(va, pb[0][u], acc[0][t]);
              acc[1][t] = Elt<T>::mfma32(va, pb[1][u], acc[1][t]);
            }
          }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();   // next tile landed; everyone is done with this one
      };
      for (int kt = 0; kt < kend; kt += 2 * BN) {
        step(kt, lds0, lds1);
        if (kt + BN < kend) step(kt + BN, lds1, lds0);
      }

#pragma unroll
      for (int rho = 0; rho < 2; ++rho) {
        const float l_tot = sum_xor16_32(l[rho]);
        if (tok[rho] < 0) continue;
        const float inv = 1.f / l_tot;
        uint16_t* orow = op + ((int64_t)tok[rho] * hq + head[rho]) * D;
#pragma unroll
        for (int t = 0; t < NT; ++t) {   // lane holds d = 16t + 4kq + r, r = 0..3
          *reinterpret_cast<u32x2_t*>(orow + 16 * t + 4 * kq) =
              u32x2_t{Elt<T>::pack2(acc[rho][t][0] * inv, acc[rho][t][1] * inv),
                      Elt<T>::pack2(acc[rho][t][2] * inv, acc[rho][t][3] * inv)};
        }
      }
    }
  }
}

template <typename T>
static hipError_t prefill_dispatch(const AttnArgs& a, int head_size, int64_t max_blocks, int num_cus,
                                  hipStream_t st) {
  const void* fn = head_size == 128 ? (const void*)&prefill_kernel<T, 128> : (const void*)&prefill_kernel<T, 64>;
  int64_t grid = resident_blocks(fn, num_cus);
  if (grid > max_blocks) grid = max_blocks;
  if (grid < 1) grid = 1;
  if (head_size == 128)
    hipLaunchKernelGGL((prefill_kernel<T, 128>), dim3((unsigned)grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_kernel<T, 64>), dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const AttnArgs& a, int dtype, int head_size, int64_t max_blocks,
                         int num_cus, hipStream_t st) {
  return dtype == 0 ? prefill_dispatch<F16>(a, head_size, max_blocks, num_cus, st)
                    : prefill_dispatch<BF16>(a, head_size, max_blocks, num_cus, st);
}

}  // namespace pa
