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
// Work item = (sequence b, KV head kh, tile): 256 query rows, row r being
// token i0 + r / G of the tile and query head kh*G + r % G, so the G heads
// that share kh share every K/V tile.  Items come from 8 per-XCD queues
// (work-group w serves queue w % 8 first, then steals from the others).
// Each of the 8 waves owns 32 rows (two 16-row groups).  Per 64-key tile:
//   K, V rows resolved through the block table (one block id per wave per
//   tile), copied HBM -> LDS by 128-bit direct-to-LDS loads into a ring of
//   four tile buffers
//   S^T = K . Q^T          16x16x32 MFMA (fp16/bf16 in, fp32 acc)
//   causal mask key <= past + i, online softmax in fp32 (exp2)
//   O^T += V^T . P^T       16x16x32 MFMA, P rounded to the input dtype
// Key tiles beyond the tile's last visible key are never loaded, and a wave
// skips the matrix work of key tiles that lie wholly above its rows'
// diagonal; the causal mask is applied only on tiles that cross a row's
// diagonal, and the output accumulators are rescaled only when a row's
// running max moves.  Key rows past the visible range are replaced by the
// last visible row, so NaN in unused cache slots never enters LDS.
#pragma once

#include <type_traits>

#include "pa_common.hpp"
#include "pa_internal.hpp"
#include "pa_lds.hpp"

namespace pa {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) short4_t* lds_s4_t;
typedef __attribute__((address_space(4))) int32_t const_i32_t;

// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4): lane l
// copies the 16 bytes at base + voff (base wave-uniform, voff a 32-bit
// per-lane byte offset) to LDS byte lds_base + 16 * l.  The compiler emits
// the SGPR-base form and sets M0 (the LDS destination) itself.  The kernel
// orders these copies with explicit vmcnt waits and barriers.  Each tick's
// __syncthreads() also waits for all of the wave's copies in flight (the
// copies write LDS); barriers that leave the newest tile's copies in flight
// measured slower, since copies landing during the matrix-core phase compete
// with its LDS operand reads.
__device__ inline void lds_dma16(const void* base, uint32_t voff, uint32_t lds_base) {
  __builtin_amdgcn_global_load_lds((const unsigned char*)base + voff,
                                   (__attribute__((address_space(3))) void*)(uintptr_t)lds_base,
                                   16, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ inline void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// K/V tiles live in LDS as unpadded rows of D halfs whose 16-byte chunks are
// XOR-swizzled by the row index, with one swizzle per operand so that both
// the row-wise K reads (kslot()) and the transposed V reads (slot()) are free
// of bank conflicts.  Tiles are
// filled by global_load_lds_dwordx4 (HBM/L2 -> LDS without registers) into a
// ring of four buffers; tile i+2 is requested four barrier ticks before it
// is first read.
//
// Eight waves, 32 query rows each, in two groups of four (one wave of each
// group per SIMD).  The groups run the same per-tile program offset by one
// phase ("ping-pong"): while group A issues the matrix-core work of a tile
// (QK^T of tile i and P.V of tile i-1), group B runs the softmax of the
// previous tile on the vector ALUs, and at the next barrier they swap, so
// the two halves of every SIMD keep the MFMA and VALU pipes busy together.
// Runs prefill work items on the calling work-group (512 threads, all of
// which must call it) until every queue is exhausted.
// CAP: scores soft-capped (c tanh(scale s / c)).  WIN: sliding window of
// a.window keys: the item's tiles start at the first one holding a key its
// first row sees, and tiles below a row's window start are masked like the
// causal diagonal.  Each option is its own instantiation, so the plain
// kernel keeps its short instruction stream and loop structure.
template <typename T, int D, bool CAP = false, bool WIN = false>
__device__ __forceinline__ void prefill_items(const AttnArgs& a) {
  constexpr int NS = D / 32;            // QK^T steps
  constexpr int NT = D / 16;            // O^T tiles
  constexpr int NR = 2;                 // 16-row groups per wave (32 rows)
  constexpr int NW = 8;                 // waves per work-group
  static_assert(kPrefillRows == 32 * NW, "tile rows");
  constexpr int BN = kPrefillKeys;      // keys per K/V tile (64)
  constexpr int NK = BN / 16;           // 16-key groups per tile
  constexpr int ROWB = D * 2;           // bytes per K/V row
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int RPI = 1024 / ROWB;      // rows per wave-wide 1 KiB LDS load
  constexpr int RPW = BN / NW;          // tile rows loaded by each wave
  constexpr int LPW = RPW / RPI;        // loads per wave per operand
  constexpr int TB = BN * ROWB;         // bytes per operand tile
  static_assert(LPW >= 1 && NK % 2 == 0, "tile shape");
  constexpr int NB = 4;                 // ring buffers of [K tile, V tile]
  __shared__ __attribute__((aligned(1024))) unsigned char lds[NB * 2 * TB];
  // The item slot lives in the decode phase's staging buffer (never in use
  // at the same time), so ring + staging fit the 160 KiB of LDS at D = 128.
  int& item_sh = *reinterpret_cast<int*>(decode_stage<T, D, CAP, WIN, 2>());
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(lds_ptr_t)lds;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;            // 0: group A, 1: group B
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

  // Slot of 16-byte chunk `chunk` of V row `row`: XOR with the row's low
  // log2(CPR) bits rotated left by one, so the transposed reads (4 rows,
  // two adjacent chunks) touch distinct slots.
  constexpr int CB = CPR == 16 ? 4 : 3;
  auto swz = [](int row) { return ((row << 1) | ((row >> (CB - 1)) & 1)) & (CPR - 1); };
  auto slot = [&](int row, int chunk) { return row * ROWB + ((chunk ^ swz(row)) << 4); };
  // Slot of 16-byte chunk `chunk` of K row `row`.  A QK^T operand read puts
  // 16 lanes on 16 consecutive rows at one chunk; the LDS serves 16 lanes of
  // a 128-bit read per pass over 64 four-byte banks, so those 16 slots must
  // differ in their bank group: XOR with row & 15 for 256-byte rows; for
  // 128-byte rows, rows of equal parity share bank halves, so (row >> 1) & 7.
  // (The V swizzle above leaves this read 2-way conflicted.)
  auto kswz = [](int row) { return CPR == 16 ? (row & 15) : ((row >> 1) & 7); };
  auto kslot = [&](int row, int chunk) { return row * ROWB + ((chunk ^ kswz(row)) << 4); };

  // Byte offsets of this wave's tile rows RPW*wave + p*RPI + ln/CPR inside
  // their cache block, with the chunk swizzles applied: constants of the
  // work-group, parked in this wave's own slice of the decode staging buffer
  // (idle in the prefill phase; no other wave touches the slice, so no
  // barrier) and read back with one LDS read per tile.  Tile t's copies add
  // a wave-uniform part (block start, and for blocks of BN keys or more the
  // tile's row offset in its block) to the scalar base, so they need no
  // vector address arithmetic.  The last tile of an item, whose rows past
  // the visible range are clamped, takes the general path.
  static_assert(2 * LPW <= 4 && 16 * ROWB >= 2048, "copy offsets slot");
  unsigned char* const offs_lds = decode_stage<T, D, CAP, WIN, 2>() + wave * (16 * ROWB) + 1024;
  {
    const int ln = lane_here();
    uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int p = 0; p < LPW; ++p) {
      const int row = RPW * wave + p * RPI + ln / CPR;
      const int rib = bsz >= BN ? row : (row & (bsz - 1));
      o[2 * p] = (uint32_t)((rib * (int)row_stride + ((ln % CPR) ^ kswz(row)) * 8) * 2);
      o[2 * p + 1] = (uint32_t)((rib * (int)row_stride + ((ln % CPR) ^ swz(row)) * 8) * 2);
    }
    *reinterpret_cast<u32x4_t*>(offs_lds + ln * 16) = u32x4_t{o[0], o[1], o[2], o[3]};
  }

  for (int qi = 0; qi < kQueues; ++qi) {
    const int x = (home + qi) % kQueues;
    // Uniform plan results: keep them in scalar registers.
    const int qlen = __builtin_amdgcn_readfirstlane(a.counters[kQueueLen + x]);
    const int qstart = __builtin_amdgcn_readfirstlane(a.counters[kQueueStart + x]);
    if (qlen == 0) continue;   // no atomics or barriers on empty queues
    for (;;) {
      if (tid == 0) item_sh = atomicAdd(a.counters_rw + kCtrPrefill + kLine * x, 1);
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
      const int n = (kend + BN - 1) / BN;      // key tiles of this item: t_lo .. n-1
      const int W = WIN ? a.window : 0;
      // first tile with a key the item's first row sees (its window start)
      const int t_lo = W > 0 ? max(0, past + i0 - W + 1) / BN : 0;
      const int nrel = n - t_lo;               // tiles processed, tick pairs 0 .. nrel
      // The block table is read-only here: read it through the constant
      // address space so uniform reads become scalar loads (tracked apart
      // from the vector-memory counter the tile copies use).
      const const_i32_t* trow =
          (const const_i32_t*)(a.block_table + (int64_t)b * a.max_blocks_per_seq);

      // Block id of this wave's RPW-row group of key tile t (rows of a
      // group never straddle a block: RPW divides the block size).
      auto block_of = [&](int t) { return trow[min(t * BN + RPW * wave, kend - 1) >> shift]; };
      // Rows [RPW*wave, RPW*wave+RPW) of the K and V tiles of key tile t;
      // keys at or past kend are clamped onto key kend-1 (finite, masked).
      auto issue = [&](int t, int blk) {
        // Block start (wave-uniform, scalar) + 32-bit lane offset in bytes.
        const int64_t bstart = (int64_t)blk * bsz * row_stride + (int64_t)kh * D;
        const uint16_t* kbase = kc + bstart;
        const uint16_t* vbase = vc + bstart;
        const uint32_t kdst = lds_addr + (uint32_t)((t % NB) * 2 * TB + RPW * wave * ROWB);
        const int ln = lane_here();   // recomputed, not held across the tile loop
#pragma unroll
        for (int p = 0; p < LPW; ++p) {
          const int row = RPW * wave + p * RPI + ln / CPR;
          const int j = min(t * BN + row, kend - 1);
          const int rof = (j & (bsz - 1)) * (int)row_stride;
          const uint32_t koff = (uint32_t)((rof + ((ln % CPR) ^ kswz(row)) * 8) * 2);
          const uint32_t voff = (uint32_t)((rof + ((ln % CPR) ^ swz(row)) * 8) * 2);
          lds_dma16(kbase, koff, kdst + p * 1024);
          lds_dma16(vbase, voff, kdst + TB + p * 1024);
        }
      };

      // The copies of a tile that is not the item's last: lane offsets held
      // (koff_l / voff_l), everything else wave-uniform.
      auto issue_fast = [&](int t, int blk) {
        const int64_t in_blk = bsz >= BN ? (int64_t)((t * BN) & (bsz - 1)) * row_stride : 0;
        const int64_t bstart = (int64_t)blk * bsz * row_stride + (int64_t)kh * D + in_blk;
        const uint16_t* kbase = kc + bstart;
        const uint16_t* vbase = vc + bstart;
        const uint32_t kdst = lds_addr + (uint32_t)((t % NB) * 2 * TB + RPW * wave * ROWB);
        const u32x4_t o = *reinterpret_cast<const u32x4_t*>(offs_lds + lane_here() * 16);
#pragma unroll
        for (int p = 0; p < LPW; ++p) {
          lds_dma16(kbase, o[2 * p], kdst + p * 1024);
          lds_dma16(vbase, o[2 * p + 1], kdst + TB + p * 1024);
        }
      };
      auto issue_tile = [&](int t, int blk) {
        if (t + 1 < n)
          issue_fast(t, blk);
        else
          issue(t, blk);
      };

      // Per-lane indices taken per item (lane_here), so values derived from
      // them are not hoisted out of the item loop and held across it.
      const int lane = lane_here();
      const int r16 = lane & 15, kq = lane >> 4;
      // Operand-read offsets.  Both swizzles XOR the chunk index with row
      // bits that are fixed per lane, so every operand read is one XOR-add on
      // two values held per lane plus an immediate offset:
      //  K, chunk 4s + kq of row 16 kap + r16 (kslot):
      //    16 kap ROWB + k_lane + (k_x ^ 64 s);
      //  V^T, d-tile t, key row 32u + 16e + vrow (vread):
      //    32u ROWB + 16e ROWB + v_lane + (v_x ^ 32 t).
      // (kswz(r16) = 4 k_x/64 + its low two bits; swz(vrow) = 2 v_x/32 + its
      // low bit; u, e and kap only move rows by multiples of 16.)
      const int ksw = kswz(r16);
      const uint32_t k_lane = (uint32_t)(r16 * ROWB + 16 * (kq ^ (ksw & 3)));
      uint32_t k_x = (uint32_t)(64 * (ksw >> 2));
      const int vrow = 4 * kq + (r16 >> 2);
      const int vsw = swz(vrow);
      const uint32_t v_lane =
          (uint32_t)(vrow * ROWB + 16 * (((lane & 3) >> 1) ^ (vsw & 1)) + ((lane & 1) << 3));
      uint32_t v_x = (uint32_t)(32 * (vsw >> 1));

      // Q^T operands and causal limits of this lane's row groups.
      u32x4_t qreg[NR][NS];
      int limit[NR];
#pragma unroll
      for (int rho = 0; rho < NR; ++rho) {
        const int row = 32 * wave + 16 * rho + r16;
        const int rg = div_small(row, a.inv_group);
        const int ti = i0 + rg;
        const bool valid = row < TQ * G && ti < ql;
        const int head = kh * G + row - rg * G;
        limit[rho] = valid ? past + ti : -1;
        const uint16_t* qrow = qp + (int64_t)(valid ? si.cu + ti : 0) * a.q_stride + (int64_t)head * D;
#pragma unroll
        for (int s = 0; s < NS; ++s)
          qreg[rho][s] = valid ? ld16(qrow + (4 * s + kq) * 8) : u32x4_t{0, 0, 0, 0};
        // Q rotated as loaded (pa_attention_rope), at the token's position.
        if (a.rope_dim > 0 && valid && past + ti < a.rope_max_pos) {
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const int e = (4 * s + kq) * 8;
            if (e < a.rope_dim)
              qreg[rho][s] = rope_chunk<T>(qreg[rho][s], qrow, e, past + ti, (const uint16_t*)a.rope_cos,
                                           (const uint16_t*)a.rope_sin, a.rope_dim, a.rope_inter != 0);
          }
        }
      }
      // Largest and smallest causal limit over this wave's rows
      // 32*wave .. 32*wave+31 (a padding row counts as -1), in closed form
      // from wave-uniform values so the per-tile branches below are
      // uniform: limits grow with the row, and rows below rows_valid are
      // the real ones.
      int wave_kmax = -1, wave_kmin = -1;
      {
        const int r0 = 32 * wave;
        const int rows_valid = min(TQ, ql - i0) * G;
        if (r0 < rows_valid) {
          wave_kmax = past + i0 + min(r0 + 31, rows_valid - 1) / G;
          if (r0 + 31 < rows_valid) wave_kmin = past + i0 + r0 / G;
        }
      }

      float m[NR], l[NR];
      float4_t acc[NR][NT];
#pragma unroll
      for (int rho = 0; rho < NR; ++rho) {
        m[rho] = -INFINITY;
        l[rho] = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[rho][t] = float4_t{0.f, 0.f, 0.f, 0.f};
      }
      float4_t sacc[NK][NR];   // scores of the tile between its M and V phases
      u32x4_t pb[NR][NK / 2];  // rounded P of the tile between its V and next M phases

      // Prologue: tiles t_lo and t_lo+1 resident, block id of the next fetched.
      issue_tile(t_lo, block_of(t_lo));
      if (nrel > 1) issue_tile(t_lo + 1, block_of(t_lo + 1));
      int blk_next = nrel > 2 ? block_of(t_lo + 2) : 0;
      wait_vmcnt<0>();
      // The wait above is opaque to the compiler, which would otherwise
      // still count the Q loads as in flight and guard their first use in
      // every tile with a full vmcnt(0) (waiting for the tile copies too).
      // Passing the operands through an empty asm marks them as ready.
#pragma unroll
      for (int rho = 0; rho < NR; ++rho)
#pragma unroll
        for (int s = 0; s < NS; ++s) asm volatile("" : "+v"(qreg[rho][s]));
      __syncthreads();

      // acc += P_t V_t with V of tile t (buffer t % 4).
      auto pv = [&](int t) {
          // O^T tile t covers d = 16t .. 16t+15.  ds_read_b64_tr_b16: within
          // each 16-lane group, result lane i gets element i % 4 of the
          // 8 bytes read by source lanes 4r + i / 4 (r = 0..3).  Source lane
          // (kq, r, q) reads key row 4kq + r at d = 16t + 4q .. +3, so lane
          // i receives d = 16t + i of keys 4kq .. 4kq+3: the V^T operand,
          // with contraction element e <-> key 32u + 4kq + e (e < 4) or
          // 32u + 16 + 4kq + (e - 4), the same keys pb holds.
          // Operands in groups of VG (u, t .. t+VG-1); group g+1 is read while
          // group g feeds its MFMAs (two register sets, fenced as in qk).
          constexpr int VG = 4;
          constexpr int NG = (NK / 2) * NT / VG;
          // v_x passes through an empty asm each tile, so the XOR stays one
          // v_xad_u32 per read instead of a table of per-lane offsets held
          // across the tile loop.
          asm volatile("" : "+v"(v_x));
          const uint32_t vb = (uint32_t)((t % NB) * 2 * TB + TB) + v_lane;
          auto vread = [&](int u, int dt) {
            const unsigned char* p = lds + ((v_x ^ (uint32_t)(32 * dt)) + vb) + 32 * u * ROWB;
            const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t)p);
            const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t)(p + 16 * ROWB));
            const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo);
            const u32x2_t h2 = __builtin_bit_cast(u32x2_t, hi);
            return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
          };
          u32x4_t va[2][VG];
#pragma unroll
          for (int e = 0; e < VG; ++e) va[0][e] = vread(0, e);
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            if (g + 1 < NG) {
#pragma unroll
              for (int e = 0; e < VG; ++e) {
                const int k = (g + 1) * VG + e;
                va[(g + 1) & 1][e] = vread(k / NT, k % NT);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < VG; ++e) {
              const int k = g * VG + e, u = k / NT, t = k % NT;
#pragma unroll
              for (int rho = 0; rho < NR; ++rho)
                acc[rho][t] = Elt<T>::mfma32(va[g & 1][e], pb[rho][u], acc[rho][t]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
      };
      // S = K_t Q^T with K of tile t.  The K operands of 16-key group kap+1
      // are read while group kap feeds its MFMAs (two register sets; the
      // fences keep each group's reads a group ahead of their use, so the
      // LDS latency hides under the previous group's 8 MFMAs).  Group 0's
      // operands are read by qk_first, which the matrix-core phase issues
      // before its P.V, so their latency hides under the P.V MFMAs; qk()
      // then reads the tile whose offsets qk_first(t) left in koff.
      u32x4_t ka[2][NS];
      uint32_t koff[NS];   // this tile's K read offsets for kap = 0 (qk_first)
      auto qk_first = [&](int t) {
        asm volatile("" : "+v"(k_x));   // one v_xad_u32 per offset, as v_x in pv
        const uint32_t kb = (uint32_t)((t % NB) * 2 * TB) + k_lane;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          koff[s] = (k_x ^ (uint32_t)(64 * s)) + kb;
          ka[0][s] = *reinterpret_cast<const u32x4_t*>(lds + koff[s]);
        }
      };
      auto qk = [&]() {
#pragma unroll
        for (int kap = 0; kap < NK; ++kap) {
          if (kap + 1 < NK) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
              ka[(kap + 1) & 1][s] =
                  *reinterpret_cast<const u32x4_t*>(lds + koff[s] + 16 * (kap + 1) * ROWB);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int rho = 0; rho < NR; ++rho)
              sacc[kap][rho] = Elt<T>::mfma32(ka[kap & 1][s], qreg[rho][s],
                                              s == 0 ? float4_t{0.f, 0.f, 0.f, 0.f} : sacc[kap][rho]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      // Soft-capped score in log2 units from the raw dot product (CAP).
      auto capf = [&](float x) {
        return a.cap_b - 2.f * a.cap_b * __builtin_amdgcn_rcpf(exp2_fast(x * a.cap_k) + 1.f);
      };
      // Softmax of tile j into P (pb), running max / sum and rescale.
      // kMasked: apply the causal mask and the window (tiles crossing a row's
      // diagonal or window start, and every tile when scale <= 0); otherwise
      // all 64 keys are visible to every row of the wave and scale > 0.
      auto softmax = [&](int j, auto masked_tag) {
        constexpr bool kMasked = decltype(masked_tag)::value;
        const int kt = j * BN;
#pragma unroll
        for (int rho = 0; rho < NR; ++rho) {
          // The running max m is raised only when a tile max exceeds it by
          // more than kMaxSlack, so P stays <= 2^kMaxSlack and rescales are
          // rare; the result is unchanged since numerator and denominator
          // share the offset.
          float mt = -INFINITY;
          if constexpr (kMasked) {
            const int low = limit[rho] - W;   // with a window, row sees keys (low, limit]
#pragma unroll
            for (int kap = 0; kap < NK; ++kap)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int key = kt + 16 * kap + 4 * kq + i;
                const float sc = CAP ? capf(sacc[kap][rho][i]) : sacc[kap][rho][i] * c;
                sacc[kap][rho][i] = key <= limit[rho] && (!WIN || key > low) ? sc : -INFINITY;
                mt = fmaxf(mt, sacc[kap][rho][i]);
              }
          } else {
#pragma unroll
            for (int kap = 0; kap < NK; ++kap)
#pragma unroll
              for (int i = 0; i < 4; ++i) mt = fmaxf(mt, sacc[kap][rho][i]);
            mt = CAP ? capf(mt) : mt * c;   // the cap is increasing: max commutes
          }
          mt = max_xor16_32(mt);
          // (While m is -inf, m + kMaxSlack is too, so any finite tile max
          // raises it.)
          const bool raise = mt > m[rho] + kMaxSlack;
          if (__any(raise)) {   // rare after the first tile
            const float m_new = raise ? fmaxf(m[rho], mt) : m[rho];
            const float base_old = m[rho] == -INFINITY ? 0.f : m[rho];
            const float base_new = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = m[rho] == -INFINITY ? 0.f : exp2_fast(base_old - base_new);
            m[rho] = m_new;
            l[rho] *= alpha;
#pragma unroll
            for (int t = 0; t < NT; ++t) scale_in_place(acc[rho][t], alpha);
          }
          // An unmasked tile shows every row of the wave all 64 of its keys,
          // so m is finite here; a masked row can still have m = -inf.
          const float base_m = !kMasked ? m[rho] : m[rho] == -INFINITY ? 0.f : m[rho];
          float sv[NK][4];
#pragma unroll
          for (int kap = 0; kap < NK; ++kap)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sv[kap][i] = kMasked ? exp2_fast(sacc[kap][rho][i] - base_m)
                           : CAP   ? exp2_fast(capf(sacc[kap][rho][i]) - base_m)
                                   : exp2_fast(fmaf(sacc[kap][rho][i], c, -base_m));
          // P rounded to the input dtype feeds P.V; the denominator sums
          // the same rounded values, straight into l.
#pragma unroll
          for (int u = 0; u < NK / 2; ++u) {
            pb[rho][u] = u32x4_t{Elt<T>::pack2(sv[2 * u][0], sv[2 * u][1]),
                                 Elt<T>::pack2(sv[2 * u][2], sv[2 * u][3]),
                                 Elt<T>::pack2(sv[2 * u + 1][0], sv[2 * u + 1][1]),
                                 Elt<T>::pack2(sv[2 * u + 1][2], sv[2 * u + 1][3])};
#pragma unroll
            for (int w = 0; w < 4; ++w) l[rho] = Elt<T>::sum2(pb[rho][u][w], l[rho]);
          }
          __builtin_amdgcn_sched_barrier(0);   // one row group at a time (registers)
        }
      };
      using Plain = std::integral_constant<bool, false>;
      using Masked = std::integral_constant<bool, true>;

      // Tiles this wave computes, relative to t_lo: a0 .. a3-1, of which
      // a0 .. a1-1 cross a row's window start (masked), a1 .. a2-1 need no
      // mask and a2 .. a3-1 cross a row's diagonal (masked).  Absolute tile
      // nw and later lie wholly above all its rows' diagonals, tiles below
      // its first row's window start hold no visible key, and tiles from nd
      // on cross the diagonal of the wave's first row; all from uniform
      // values (wave_kmax / wave_kmin: last / first row's causal limit).
      int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
      if constexpr (!WIN) {
        a3 = wave_kmax < 0 ? 0 : min(n, wave_kmax / BN + 1);
        a2 = c > 0.f ? min(a3, (wave_kmin + 1) / BN) : 0;
      } else {
        const int nw = wave_kmax < 0 ? 0 : min(n, wave_kmax / BN + 1);
        const int nd = c > 0.f ? min(nw, (wave_kmin + 1) / BN) : 0;
        const int first_lim = past + i0 + 32 * wave / G;          // the wave's first row
        const int tA0 = W > 0 ? max(0, first_lim - W + 1) / BN : 0;
        const int tA1 = W > 0 ? (max(0, wave_kmax - W + 1) + BN - 1) / BN : 0;
        const int A0 = max(t_lo, min(tA0, nw));
        if (nw > A0) {
          const int A1 = min(max(tA1, A0), nw);
          const int A2 = min(max(nd, A1), nw);
          a0 = A0 - t_lo;
          a1 = A1 - t_lo;
          a2 = A2 - t_lo;
          a3 = nw - t_lo;
        }
      }

      // Request tile i+2: issued by each wave at the start of its softmax
      // phase (group B: tick 2i, group A: tick 2i+1).  Issuing 32 copies at
      // once can stall the issuing waves until the address unit drains them,
      // which must not happen in a matrix-core phase.
      auto even_service = [&](int i) {
        if (i + 2 < nrel) issue_tile(t_lo + i + 2, blk_next);
      };
      // Block id of tile i+3 (a scalar load, first used at tick 2i+2), read
      // at the start of the wave's softmax phase: that phase has no LDS reads
      // and hides the load, whereas an SMEM load in flight during the
      // matrix-core phase would turn its LDS waits into full lgkmcnt drains.
      auto fetch_service = [&](int i) {
        if (i + 3 < nrel) blk_next = block_of(t_lo + i + 3);
      };
      // Run at the end of tick 2i+1 by every wave, before its barrier: all
      // copies but tile i+2's have landed, so tile i+1 is complete.
      auto odd_service = [&](int i) {
        if (i + 2 < nrel) wait_vmcnt<2 * LPW>(); else wait_vmcnt<0>();
      };

      // Tick pair i (ticks 2i and 2i+1) of tile t = t_lo + i: ticks 2i and
      // 2i+1 request tile t+2; tick 2i+1 ends with tile t+1 complete.  Tile t
      // lives in ring buffer t % 4: tile t+2 overwrites tile t-2, whose V was
      // last read at tick 2i-1.
      // Group A runs M_i = {P.V of tile t-1, QK^T of tile t} at tick 2i and
      // the softmax V_i at tick 2i+1; group B runs V_{i-1} at tick 2i and
      // M_i at tick 2i+1.  Both pass the same 2(nrel+1) barriers; a wave
      // idles through the pairs outside a0 .. a3, and the loops are split
      // where its tiles change kind so each body is straight-line.
      auto idle = [&](int i) {
        __syncthreads();
        even_service(i);
        fetch_service(i);
        odd_service(i);
        __syncthreads();
      };
      if (grp == 0) {
        auto tick = [&](int i, auto kind) {
          qk_first(t_lo + i);
          __builtin_amdgcn_sched_barrier(0);
          if (i > a0) pv(t_lo + i - 1);
          __builtin_amdgcn_sched_barrier(0);
          qk();
          __syncthreads();
          even_service(i);
          fetch_service(i);
          softmax(t_lo + i, kind);
          odd_service(i);
          __syncthreads();
        };
        int i = 0;
        if constexpr (WIN) {   // (a0 = a1 = 0 without a window)
          for (; i < a0; ++i) idle(i);
          for (; i < a1; ++i) tick(i, Masked{});
        }
        for (; i < a2; ++i) tick(i, Plain{});
        for (; i < a3; ++i) tick(i, Masked{});
        for (; i <= nrel; ++i) {
          if (i == a3 && a3 > a0) pv(t_lo + i - 1);
          idle(i);
        }
      } else {
        int i = 0;
        if constexpr (WIN)
          for (; i < a0; ++i) idle(i);
        // Tick pair a0: M_a0 = QK^T of the wave's first tile only.
        even_service(i);
        fetch_service(i);
        __syncthreads();
        if (a3 > a0) {
          qk_first(t_lo + i);
          qk();
        }
        odd_service(i);
        __syncthreads();
        ++i;
        auto tick = [&](int i, auto kind) {   // V_{i-1}, then M_i
          even_service(i);
          fetch_service(i);
          softmax(t_lo + i - 1, kind);
          __syncthreads();
          qk_first(t_lo + i);
          __builtin_amdgcn_sched_barrier(0);
          pv(t_lo + i - 1);
          __builtin_amdgcn_sched_barrier(0);
          qk();
          odd_service(i);
          __syncthreads();
        };
        if constexpr (WIN)
          for (; i < min(a1 + 1, a3); ++i) tick(i, Masked{});
        for (; i < min(a2 + 1, a3); ++i) tick(i, Plain{});
        for (; i < a3; ++i) tick(i, Masked{});
        if (i == a3 && a3 > a0) {   // V of the last tile (masked: a no-op on a plain one), P.V only
          even_service(i);
          fetch_service(i);
          softmax(t_lo + i - 1, Masked{});
          __syncthreads();
          pv(t_lo + i - 1);
          odd_service(i);
          __syncthreads();
          ++i;
        }
        for (; i <= nrel; ++i) idle(i);
      }

      // Output rows: token and head recomputed here (not held in registers
      // through the tile loops).
      const int eln = lane_here();
#pragma unroll
      for (int rho = 0; rho < NR; ++rho) {
        const float l_tot = sum_xor16_32(l[rho]);
        if (limit[rho] < 0) continue;   // padding row
        const float inv = 1.f / l_tot;
        const int row = 32 * wave + 16 * rho + (eln & 15);
        const int rg = div_small(row, a.inv_group);
        const int64_t orow_el = ((int64_t)(si.cu + i0 + rg) * hq + kh * G + row - rg * G) * D;
        uint16_t* orow = op + orow_el + 4 * (eln >> 4);
#pragma unroll
        for (int t = 0; t < NT; ++t) {   // lane holds d = 16t + 4kq + r, r = 0..3
          *reinterpret_cast<u32x2_t*>(orow + 16 * t) =
              u32x2_t{Elt<T>::pack2(acc[rho][t][0] * inv, acc[rho][t][1] * inv),
                      Elt<T>::pack2(acc[rho][t][2] * inv, acc[rho][t][3] * inv)};
        }
      }
    }
  }
}

}  // namespace pa
