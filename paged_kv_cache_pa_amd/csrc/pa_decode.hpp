// Decode path: split-KV paged attention for sequences whose q_len * G query
// columns fit one 16-wide tile (q_len == 1 decode, and short speculative
// chunks), plus the log-sum-exp combine of the splits.
//
// Sources: "[WebGPU] Initial PagedAttention implementation (1/n)" -
// "Description" (attention over the paged cache for packed varlen queries),
// "FlashAttention: optional seqlens_q input" (past_b = total_kv_b - q_len_b;
// row i sees keys 0..past_b+i) and "Roadmap" (phase 2: page-aware decode
// reading K/V through the block table instead of a gather pass);
// FlexAttention operator page - "FlexAttention Computation" and "Grouped
// Query Attention (GQA)".
//
// Work item = (sequence b, split s, KV head kh), one wavefront each, fetched
// from a device counter.  The wave walks 16-key chunks of keys
// [s*S, min(L, (s+1)*S)), S = the split length, through the block table (the split's block ids
// are prefetched into two VGPRs and broadcast per chunk with readlane).  The
// G query heads of kh (times q_len tokens) are the 16 columns n = i*G + g of
// the score tile, so every K/V byte is read from HBM exactly once per call.
//
//   S^T[key][n] = K_chunk . Q^T       16x16x32 MFMA, D/32 steps
//   online softmax per column n       fp32, exp2 with log2(e) folded in
//   O^T[d][n]  += V_chunk^T . P^T      16x16x16 MFMA, D/16 tiles
//
// Lane (kq = l/16, r = l%16) uses, per chunk, 64 B of key row r (the A
// operand of S^T: contraction elements = 16-byte chunks 4s+kq of the row)
// and 16 B of each of value rows 4kq..4kq+3 (d range [r*D/16, (r+1)*D/16)),
// so V needs only register permutes to become the A operand of O^T: tile t
// row r stands for d = r*D/16 + t.  Every load instruction covers whole
// cache rows: the V loads do as they stand; K is loaded with the lanes along
// its rows and turned into the operand layout through a per-wave LDS slice
// (a CU streams whole-row loads about twice as fast as the operand shape,
// 16 rows x 64 B, when few CUs stream).  K and V take non-temporal loads.
// The accumulator tile of O^T keeps column n in lane n%16, the same lane
// that owns column n's softmax state, so rescaling is a per-lane multiply.
//
// A sequence with one split writes its normalised output directly; longer
// sequences write (m, l, unnormalised acc) per split and column, merged by
// combine_kernel:  O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
//
// fp8 caches (KV8; e4m3 elements with a float32 scale per KV head and
// channel, the quantized KV cache of the "Roadmap", phase 3): the same
// matrix-core program on half the bytes.  A lane's K bytes are made
// contiguous by giving lane group kq the contraction chunks NS*kq .. +NS-1
// (Q^T loaded with the same chunk order), so a lane uses 8*NS bytes of its
// key row (staged as above) and loads NT bytes of each of its four value
// rows.  Chunks stay as raw
// bytes in flight and are widened to fp16/bf16 (exact) just before their
// MFMAs.  The K scale of channel d multiplies q_d once per item (in fp32,
// then rounded to the MFMA type with the rest of Q^T); the V scale
// multiplies the accumulators before they are stored.
#pragma once

#include <type_traits>

#include "pa_common.hpp"
#include "pa_internal.hpp"
#include "pa_lds.hpp"

namespace pa {

// Runs decode work items on the calling wave until the decode counter is
// exhausted.  Every wave is independent (no barriers, no LDS).
// CAP / WIN: the score soft cap / the sliding window is on (compile-time, so
// the plain score loop carries no selects for them).
template <typename T, int D, bool KV8 = false, bool CAP = false, bool WIN = false>
__device__ __forceinline__ void decode_items(const AttnArgs& a) {
  constexpr int NS = D / 32;    // QK^T contraction steps (8 halfs per lane)
  constexpr int NT = D / 16;    // O^T tiles; also halfs per lane per V row
  // Lane from lane_here() rather than threadIdx: each inlined copy of this
  // body then derives its own per-lane values, instead of sharing values
  // computed once at kernel entry that would stay live (spilled) across the
  // other work the kernel does in between.
  const int lane = lane_here();
  const int r16 = lane & 15, kq = lane >> 4;
  const int hk = a.num_kv_heads, G = a.group, hq = a.num_heads;
  const int64_t row_stride = (int64_t)hk * D;   // elements between token rows
  const uint16_t* __restrict__ qp = (const uint16_t*)a.q;
  typedef typename std::conditional<KV8, uint8_t, uint16_t>::type CT;   // cache element
  const CT* __restrict__ kc = (const CT*)a.k_cache;
  const CT* __restrict__ vc = (const CT*)a.v_cache;
  uint16_t* __restrict__ op = (uint16_t*)a.out;
  const int n_items = a.counters[kNumDecPairs] * hk;

  for (;;) {
    int it = 0;
    if (lane == 0) it = atomicAdd(a.counters_rw + kCtrDecode, 1);
    it = __builtin_amdgcn_readfirstlane(__shfl(it, 0));
    if (it >= n_items) return;
    const int pair = it / hk;
    const int kh = it - pair * hk;
    const int2 bsplit = a.dec_items[pair];
    const int b = bsplit.x, split = bsplit.y;
    const SeqInfo si = a.seqinfo[b];
    const int L = si.kv_len, ql = si.q_len;
    const int past = L - ql;
    const int ncols = ql * G;
    const int nsplit = (L + a.split_keys - 1) >> a.split_shift;
    const int live = nsplit - (WIN ? first_live_split(L, ql, a.window, a.split_shift) : 0);   // splits with items
    const int k0 = split << a.split_shift;
    const int k1 = min(L, k0 + a.split_keys);

    // Q^T operand: column n = r16 -> (token n / G, head kh*G + n % G).
    u32x4_t qreg[NS];
    {
      const int n = r16;
      const bool valid = n < ncols;
      const int ng = div_small(n, a.inv_group);
      const int tok = si.cu + (valid ? ng : 0);
      const int h = kh * G + (valid ? n - ng * G : 0);
      const uint16_t* qrow = qp + (int64_t)tok * a.q_stride + (int64_t)h * D;
      if constexpr (!KV8) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          qreg[s] = valid ? ld16(qrow + (4 * s + kq) * 8) : u32x4_t{0, 0, 0, 0};
        }
        // Q rotated as loaded (pa_attention_rope), at the token's position.
        const int pos = past + ng;
        if (a.rope_dim > 0 && valid && pos < a.rope_max_pos) {
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const int e = (4 * s + kq) * 8;
            if (e < a.rope_dim)
              qreg[s] = rope_chunk<T>(qreg[s], qrow, e, pos, (const uint16_t*)a.rope_cos,
                                      (const uint16_t*)a.rope_sin, a.rope_dim, a.rope_inter != 0);
          }
        }
      } else {
        const float* ks = a.k_scale + (int64_t)kh * D;
        // Q rotated as loaded (pa_attention_rope_fp8) and rounded to the
        // input dtype, as the rotary scatter's q_out would hold it, before
        // the K scale is applied.
        const int pos = past + ng;
        const bool rot = a.rope_dim > 0 && valid && pos < a.rope_max_pos;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int d0 = (NS * kq + s) * 8;
          u32x4_t x = ld16(qrow + d0);
          if (rot && d0 < a.rope_dim)
            x = rope_chunk<T>(x, qrow, d0, pos, (const uint16_t*)a.rope_cos,
                              (const uint16_t*)a.rope_sin, a.rope_dim, a.rope_inter != 0);
          const float4_t s0 = *reinterpret_cast<const float4_t*>(ks + d0);
          const float4_t s1 = *reinterpret_cast<const float4_t*>(ks + d0 + 4);
          const float2 f0 = Elt<T>::unpack2(x[0]), f1 = Elt<T>::unpack2(x[1]);
          const float2 f2 = Elt<T>::unpack2(x[2]), f3 = Elt<T>::unpack2(x[3]);
          const u32x4_t y = {Elt<T>::pack2(f0.x * s0[0], f0.y * s0[1]),
                             Elt<T>::pack2(f1.x * s0[2], f1.y * s0[3]),
                             Elt<T>::pack2(f2.x * s1[0], f2.y * s1[1]),
                             Elt<T>::pack2(f3.x * s1[2], f3.y * s1[3])};
          qreg[s] = valid ? y : u32x4_t{0, 0, 0, 0};
        }
      }
    }
    // Causal limit of column n: token n / G sees keys <= past + n / G
    // (padding columns see every key and are never stored); with a sliding
    // window W it sees only keys > col_limit - W.
    const int col_limit = past + div_small(r16, a.inv_group);
    const int col_low = col_limit - (WIN ? a.window : 0);

    // Block ids of this split: block i in lane i % 64 of register i / 64
    // (a split spans at most 128 blocks).
    const int blk0 = k0 >> a.block_shift;
    const int nblk = ((k1 - 1) >> a.block_shift) - blk0 + 1;
    const int32_t* trow = a.block_table + (int64_t)b * a.max_blocks_per_seq + blk0;
    const int my_blk = lane < nblk ? trow[lane] : 0;
    const int my_blk2 = lane + 64 < nblk ? trow[lane + 64] : 0;

    float m = -INFINITY, l = 0.f;
    float4_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

    // K/V registers of one 16-key chunk, as loaded: 16-bit elements, or fp8
    // codes (KV8: NS/2 16-byte K loads and NT/4 dwords per value row).
    constexpr int KW = KV8 ? NS / 2 : NS;
    constexpr int VW = KV8 ? NT / 4 : NT / 2;
    // K is loaded in whole rows: each wave-wide load covers KRPI complete
    // key rows (one 16-byte chunk per lane).  The matrix-core operand wants
    // the other shape (16 rows x 64 bytes per load: half of 16 different
    // 128-byte lines), and a CU streams that shape at about half the rate:
    // a probe measured 80 vs 38 GB/s per CU on 16-32 CUs, 37.5 vs 33.7 on
    // 128.  The chunk is turned into the operand layout through this wave's
    // own 16-row LDS slice (XOR-swizzled so the 16-row reads and the row
    // writes are conflict-free).  V loads already cover whole rows.
    constexpr int KROWB = D * (int)sizeof(CT);     // bytes per K row
    constexpr int KCPR = KROWB / 16;               // 16-byte chunks per row
    constexpr int KRPI = 64 / KCPR;                // rows per wave-wide load
    static_assert(16 / KRPI == KW && 8 * 16 * KROWB == decode_stage_bytes<D, sizeof(CT)>(),
                  "K staging");
    constexpr int KRP = 256 / KROWB;               // rows per 256 bytes (64 banks)
    auto kswz = [](int row) { return (row / KRP) & (KCPR - 1); };
    unsigned char* const kst =
        decode_stage<T, D, CAP, WIN, (int)sizeof(CT)>() +
        __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * (16 * KROWB);
    struct Chunk {
      u32x4_t k[KW];
      uint32_t v[4][VW];
    };
    auto load = [&](int c0, Chunk& ch) {
      const int bi = (c0 >> a.block_shift) - blk0;   // uniform
      const int blk = bi < 64 ? __builtin_amdgcn_readlane(my_blk, bi)
                              : __builtin_amdgcn_readlane(my_blk2, bi - 64);
      const int64_t base =
          ((int64_t)blk * a.block_size + (c0 & (a.block_size - 1))) * row_stride + (int64_t)kh * D;
      // Load j: rows j * KRPI .. + KRPI - 1, chunk lane % KCPR of row
      // j * KRPI + lane / KCPR.  K and V stream through once, so both take
      // non-temporal loads: with every cache line requested by exactly one
      // load, pure decode is 7 % faster and the mixed batch 2 % (with the
      // older half-line K loads, where a line's second request relied on
      // the L2, the same hint made the mixed batch 4 % slower).
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        const int row = j * KRPI + lane / KCPR;
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
            reinterpret_cast<const unsigned char*>(kc + base + row * row_stride) +
            (lane % KCPR) * 16);
        ch.k[j] = __builtin_nontemporal_load(src);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const CT* vrow = vc + base + (4 * kq + e) * row_stride + r16 * NT;
        if constexpr (VW == 4) {
          const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vrow));
#pragma unroll
          for (int w = 0; w < 4; ++w) ch.v[e][w] = x[w];
        } else if constexpr (VW == 2) {
          const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(vrow));
#pragma unroll
          for (int w = 0; w < 2; ++w) ch.v[e][w] = x[w];
        } else {   // fp8 caches, head_size 64
          ch.v[e][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vrow));
        }
      }
    };
    // The chunk's K in the operand layout: piece j of lane (r16, kq) is
    // 16-byte chunk 4j + kq (16-bit; 8 elements, QK^T step j) or KW kq + j
    // (fp8; 16 codes, steps 2j and 2j+1) of key row r16.  Written as loaded,
    // then read back, by this wave alone (in order, so no barrier).
    auto k_pieces = [&](const Chunk& ch, u32x4_t (&kp)[KW]) {
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        const int row = j * KRPI + lane / KCPR, chunk = lane % KCPR;
        *reinterpret_cast<u32x4_t*>(kst + row * KROWB + ((chunk ^ kswz(row)) << 4)) = ch.k[j];
      }
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        const int chunk = KV8 ? KW * kq + j : 4 * j + kq;
        kp[j] = *reinterpret_cast<const u32x4_t*>(kst + r16 * KROWB +
                                                  ((chunk ^ kswz(r16)) << 4));
      }
    };
    // Operand of QK^T step s: 8 elements of the lane's key row.
    auto k_operand = [&](const u32x4_t (&kp)[KW], int s) -> u32x4_t {
      if constexpr (!KV8) {
        return kp[s];
      } else {
        const uint32_t lo = kp[s >> 1][2 * (s & 1)], hi = kp[s >> 1][2 * (s & 1) + 1];
        return u32x4_t{Elt<T>::template from_fp8x2<0>(lo), Elt<T>::template from_fp8x2<1>(lo),
                       Elt<T>::template from_fp8x2<0>(hi), Elt<T>::template from_fp8x2<1>(hi)};
      }
    };
    // Dword w (two elements) of value row e, as 16-bit elements.
    auto v_word = [&](const Chunk& ch, int e, int w) -> uint32_t {
      if constexpr (!KV8) {
        return ch.v[e][w];
      } else {
        const uint32_t x = ch.v[e][w >> 1];
        return (w & 1) ? Elt<T>::template from_fp8x2<1>(x) : Elt<T>::template from_fp8x2<0>(x);
      }
    };
    auto compute = [&](int c0, const Chunk& ch) {
      u32x4_t kp[KW];
      k_pieces(ch, kp);
      float4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) sc = Elt<T>::mfma32(k_operand(kp, s), qreg[s], sc);
      float sv[4];
      float cmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = c0 + 4 * kq + i;
        bool vis = key < k1 && key <= col_limit;
        if constexpr (WIN) vis = vis && key > col_low;
        // soft cap: c tanh(scale s / c), in log2 units (see AttnArgs)
        const float s2 = CAP ? a.cap_b - 2.f * a.cap_b *
                                              __builtin_amdgcn_rcpf(exp2_fast(sc[i] * a.cap_k) + 1.f)
                                : sc[i] * a.scale_log2;
        sv[i] = vis ? s2 : -INFINITY;
        cmax = fmaxf(cmax, sv[i]);
      }
      cmax = max_xor16_32(cmax);
      // Raise the running max only when this chunk exceeds it by more than
      // kMaxSlack (P stays <= 2^kMaxSlack), so the accumulators are rescaled
      // rarely; numerator and denominator share the offset.
      const bool raise = cmax > m + kMaxSlack || m == -INFINITY;
      if (__any(raise)) {
        const float m_new = raise ? fmaxf(m, cmax) : m;
        const float base_new = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = m == -INFINITY ? 0.f : exp2_fast(m - base_new);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) scale_in_place(acc[t], alpha);
      }
      const float base_m = m == -INFINITY ? 0.f : m;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = exp2_fast(sv[i] - base_m);
      // P enters P.V rounded to the input dtype; the denominator sums the
      // same rounded values so the weights of each column sum to one.
      const u32x2_t pb = {Elt<T>::pack2(p[0], p[1]), Elt<T>::pack2(p[2], p[3])};
      l += Elt<T>::sum2(pb[1], Elt<T>::sum2(pb[0], 0.f));
      // Value rows at or past the split end may be unused slots (NaN).
      uint32_t vz[4][NT / 2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool live = c0 + 4 * kq + e < k1;
#pragma unroll
        for (int w = 0; w < NT / 2; ++w) vz[e][w] = live ? v_word(ch, e, w) : 0u;
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t w0 = pair_elem(vz[0][t >> 1], vz[1][t >> 1], t & 1);
        const uint32_t w1 = pair_elem(vz[2][t >> 1], vz[3][t >> 1], t & 1);
        acc[t] = Elt<T>::mfma16(u32x2_t{w0, w1}, pb, acc[t]);
      }
    };

    // Software pipeline over two register sets: chunk c+1 is requested
    // before chunk c is computed.  The loop runs over chunk pairs with a
    // uniform trip count and its only exit is the loop test, so its body is
    // straight-line and the compiler's wait counts keep the younger chunk in
    // flight; the pair's second request past the split end re-reads the
    // split's last chunk (cached) instead of branching.  A deeper ring (3 or
    // 4 chunks) measured no faster: a CU's streaming rate is bounded by its
    // outstanding-miss capacity (hence the whole-row K loads above), not by
    // how far ahead each wave issues.
    const int nch = (k1 - k0 + 15) >> 4;
    const int last_c0 = k0 + 16 * (nch - 1);
    Chunk ca, cb;
    load(k0, ca);
    for (int pr = 0; pr < (nch >> 1); ++pr) {
      const int c0 = k0 + 32 * pr;
      load(c0 + 16, cb);
      compute(c0, ca);
      load(min(c0 + 32, last_c0), ca);
      compute(c0 + 16, cb);
    }
    if (nch & 1) compute(last_c0, ca);

    const float l_tot = sum_xor16_32(l);
    if constexpr (KV8) {   // V scale of channel d = (4kq + r) * NT + t
      const float* vs = a.v_scale + (int64_t)kh * D;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < NT; t += 4) {
          const float4_t f = *reinterpret_cast<const float4_t*>(vs + (4 * kq + r) * NT + t);
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[t + u][r] *= f[u];
        }
    }
    const int n = r16;
    if (n >= ncols) {
      // padding column: nothing to store
    } else if (live == 1) {
      const float inv = 1.f / l_tot;
      const int ng = div_small(n, a.inv_group);
      const int tok = si.cu + ng;
      const int h = kh * G + n - ng * G;
      uint16_t* orow = op + ((int64_t)tok * hq + h) * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t w[NT / 2];
#pragma unroll
        for (int t = 0; t < NT; t += 2)
          w[t / 2] = Elt<T>::pack2(acc[t][r] * inv, acc[t + 1][r] * inv);
        uint16_t* dst = orow + (4 * kq + r) * NT;
        if constexpr (NT == 8) {
          *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{w[0], w[1], w[2], w[3]};
        } else {
          *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{w[0], w[1]};
        }
      }
    } else {
      const int64_t row = (int64_t)si.pbase + ((int64_t)kh * nsplit + split) * ncols + n;
      if (kq == 0) a.part_ml[row] = make_float2(m, l_tot);
      float* dst = a.part_acc + row * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float tmp[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) tmp[t] = acc[t][r];
#pragma unroll
        for (int t = 0; t < NT; t += 4)
          *reinterpret_cast<float4_t*>(dst + (4 * kq + r) * NT + t) =
              float4_t{tmp[t], tmp[t + 1], tmp[t + 2], tmp[t + 3]};
      }
    }
  }
}

// One work-group per (sequence, KV head); a no-op unless the sequence took
// the decode path with more than one split.  Per column: M = max_s m_s,
// w_s = 2^(m_s - M), and the output is sum_s w_s acc_s / sum_s w_s l_s.
// The kernel's time is its chain of dependent memory round trips, so each
// column's (m, l) pairs are loaded once, held in registers while the max is
// taken, and the partials follow eight splits per round trip.  All
// work-groups of a large batch fit on the chip at once only while the kernel
// stays near 64 registers, so nothing more is held.
constexpr int kCombineThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(AttnArgs a) {
  constexpr int MAXS = kMaxSplitsCombine;
  constexpr int MLR = 2;     // (m, l) pairs per weight lane held in registers
  constexpr int DEPTH = 8;   // partial loads in flight per thread
  __shared__ float wts[kDecodeCols][MAXS];
  __shared__ float inv_den[kDecodeCols];
  const int b = blockIdx.x, kh = blockIdx.y;
  const SeqInfo si = a.seqinfo[b];
  const int G = a.group;
  const int ncols = si.q_len * G;
  if (si.q_len <= 0 || ncols > kDecodeCols || a.force_prefill) return;
  const int nsplit = (si.kv_len + a.split_keys - 1) >> a.split_shift;
  const int s0 = first_live_split(si.kv_len, si.q_len, a.window, a.split_shift);   // splits s0 .. nsplit-1
  if (nsplit - s0 <= 1) return;
  const int64_t row0 = (int64_t)si.pbase + (int64_t)kh * nsplit * ncols;
  const int tid = threadIdx.x;

  // Column c's weights: the 16 lanes of one group; split s0 + lane16 + 16j
  // in register j, further splits (past 16 * MLR) loaded again.
  const int c = tid >> 4, lane16 = tid & 15;
  if (c < ncols) {
    auto ml_at = [&](int s) { return a.part_ml[row0 + (int64_t)s * ncols + c]; };
    float2 ml[MLR];
#pragma unroll
    for (int j = 0; j < MLR; ++j) {
      const int s = s0 + lane16 + 16 * j;
      ml[j] = s < nsplit ? ml_at(s) : make_float2(-INFINITY, 0.f);
    }
    float M = -INFINITY;
    for (int s = s0 + lane16 + 16 * MLR; s < nsplit; s += 16) M = fmaxf(M, ml_at(s).x);
#pragma unroll
    for (int j = 0; j < MLR; ++j) M = fmaxf(M, ml[j].x);
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 16));
    float den = 0.f;
    auto weigh = [&](int s, float2 v) {
      const float w = v.x == -INFINITY ? 0.f : exp2_fast(v.x - M);
      wts[c][s] = w;
      den += w * v.y;
    };
#pragma unroll
    for (int j = 0; j < MLR; ++j) {
      const int s = s0 + lane16 + 16 * j;
      if (s < nsplit) weigh(s, ml[j]);
    }
    for (int s = s0 + lane16 + 16 * MLR; s < nsplit; s += 16) weigh(s, ml_at(s));
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) den += __shfl_xor(den, o, 16);
    if (lane16 == 0) inv_den[c] = 1.f / den;
  }
  __syncthreads();

  // Each thread: 4 consecutive outputs of one column from 16-byte partial
  // loads, splits summed in order.
  uint16_t* __restrict__ op = (uint16_t*)a.out;
  const int64_t step = (int64_t)ncols * D;     // floats between one column's splits
  for (int idx = tid; idx < ncols * (D / 4); idx += kCombineThreads) {
    const int n = idx / (D / 4), d = (idx - n * (D / 4)) * 4;
    const float* src = a.part_acc + (row0 + n) * D + d;
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = s0; s < nsplit; s += DEPTH) {
      float4_t v[DEPTH];
#pragma unroll
      for (int u = 0; u < DEPTH; ++u)
        v[u] = s + u < nsplit ? *reinterpret_cast<const float4_t*>(src + (s + u) * step)
                              : float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < DEPTH; ++u)
        if (s + u < nsplit) acc += wts[n][s + u] * v[u];
    }
    const float4_t o = acc * inv_den[n];
    const int tok = si.cu + n / G;
    const int h = kh * G + n % G;
    *reinterpret_cast<u32x2_t*>(op + ((int64_t)tok * a.num_heads + h) * D + d) =
        u32x2_t{Elt<T>::pack2(o[0], o[1]), Elt<T>::pack2(o[2], o[3])};
  }
}

}  // namespace pa
