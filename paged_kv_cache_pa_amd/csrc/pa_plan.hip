// Plan: turn the device-resident varlen metadata into work lists, without
// any device-to-host copy.
//
// Source: "[WebGPU] Initial PagedAttention implementation (1/n)", section
// "FlashAttention: optional seqlens_q input" (per-sequence past length =
// total KV length - that sequence's query length) and the maintainer's note
// that the host-side metadata readback blocks every run; here the host only
// sizes the grids from host-known bounds and one work-group derives the rest.
//
// Per sequence b: q_len = cu[b+1] - cu[b], L = seqlens_kv[b].  A sequence
// whose q_len * G columns fit one 16-wide tile takes the decode path and is
// split into ceil(L / split_keys) key ranges: the decode work list holds
// every full split, then the partial last splits, longest first (by length
// class), so the work ends on the shortest items; every other non-empty
// sequence takes the prefill path in tiles of tokens_per_tile tokens per KV
// head.
// Prefill (sequence, KV head) pairs are dealt to 8 queues, one per XCD, so
// all tiles that reuse one K/V stream share an L2; inside a queue the
// heaviest (last) tile of each pair comes first.  The plan also splits the
// attention kernel's work-groups between the two kinds of work in proportion
// to their estimated CU time (prefill: 64-key tile steps x kPrefillStepCost;
// decode: key rows streamed).
#include "pa_common.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

// Block-wide exclusive scan of W ints per thread (1024 threads).
template <int W>
__device__ void block_scan(int (&v)[W], int (&total)[W], int* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc[W];
#pragma unroll
  for (int k = 0; k < W; ++k) {
    int x = v[k];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    inc[k] = x;
  }
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < W; ++k) lds[wave * W + k] = inc[k];
  }
  __syncthreads();
  if (threadIdx.x < W) {
    int run = 0;
    for (int w = 0; w < kPlanWaves; ++w) {
      int t = lds[w * W + threadIdx.x];
      lds[w * W + threadIdx.x] = run;
      run += t;
    }
    lds[kPlanWaves * W + threadIdx.x] = run;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < W; ++k) {
    v[k] = lds[wave * W + k] + inc[k] - v[k];
    total[k] = lds[kPlanWaves * W + k];
  }
  __syncthreads();
}

struct SeqCounts {
  int cu0, q_len, L, nsplit, prows, ntiles, s0;
};

__device__ inline SeqCounts seq_counts(const PlanArgs& a, int b) {
  SeqCounts c{0, 0, 0, 0, 0, 0, 0};
  if (b >= a.num_seqs) return c;
  c.cu0 = a.cu_seqlens_q[b];
  c.q_len = a.cu_seqlens_q[b + 1] - c.cu0;
  c.L = a.seqlens_kv[b];
  if (c.q_len <= 0) return c;
  const int ncols = c.q_len * a.group;
  if (a.decode_only && ncols > kDecodeCols) return c;   // no work (precondition violated)
  if (ncols <= kDecodeCols && !a.force_prefill) {
    c.nsplit = (c.L + a.split_keys - 1) >> a.split_shift;
    c.s0 = first_live_split(c.L, c.q_len, a.window, a.split_shift);
    if (c.nsplit - c.s0 > 1) c.prows = a.num_kv_heads * c.nsplit * ncols;
  } else {
    c.ntiles = (c.q_len + a.tokens_per_tile - 1) / a.tokens_per_tile;
  }
  return c;
}

// Length class of a sequence's partial last split (its L mod split keys):
// 0 for the shortest quarter of split lengths, up to 3 for the longest.
__device__ inline int part_class(int L, int split_shift) {
  return ((L & ((1 << split_shift) - 1)) << 2) >> split_shift;
}

// Number of KV heads kh in [0, Hk) with (b * Hk + kh) % 8 == x.
__device__ inline int heads_in_queue(int b, int hk, int x) {
  const int r = ((x - (int)(((int64_t)b * hk) & 7)) % 8 + 8) % 8;
  return r < hk ? (hk - 1 - r) / 8 + 1 : 0;
}

// The second-pass writes of sequence b (lane-owned values, the whole wave
// cooperating): its partial last decode split, placed after all full splits,
// and its prefill items, heaviest tile of each (sequence, KV head) first.
// part_at: slot of b's partial split; qpos[x]: first slot of b's items in
// queue x (queue start + items of earlier sequences).
__device__ inline void emit_second_pass(const PlanArgs& a, int b, const SeqCounts& c, bool has_part,
                                        int part_at, const int (&qpos)[kQueues]) {
  if (has_part) a.dec_items[part_at] = make_int2(b, c.nsplit - 1);
  // A prefill sequence's Hk x ntiles items are written by its whole wave
  // (the owning lane's values broadcast): one lane storing them in turn
  // held the plan at ~25 us on a few long prefill chunks.
  unsigned long long todo = __ballot(c.ntiles > 0);
  while (todo) {
    const int src = __builtin_ctzll(todo);
    todo &= todo - 1;
    const int bb = __shfl(b, src), nt = __shfl(c.ntiles, src);
    int vx[kQueues];
#pragma unroll
    for (int x = 0; x < kQueues; ++x) vx[x] = __shfl(qpos[x], src);
    for (int i = threadIdx.x & 63; i < a.num_kv_heads * nt; i += 64) {
      const int kh = i / nt, r = i - kh * nt;
      const int x = (int)(((int64_t)bb * a.num_kv_heads + kh) & 7);
      int pos = 0;   // first item of (bb, kh) in queue x
#pragma unroll
      for (int q = 0; q < kQueues; ++q)
        if (q == x) pos = vx[q] + (kh >> 3) * nt;
      a.pf_items[pos + r] = make_int4(bb, kh, nt - 1 - r, 0);
    }
  }
}

}  // namespace

// Partial last splits are placed longest first, in kPartClasses classes of
// their key count, so the decode work ends on the shortest items.
constexpr int kPartClasses = 4;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int lds[(kPlanWaves + 1) * 16];
  __shared__ int qstart[kQueues];
  __shared__ int part_start[kPartClasses];
  __shared__ float cost_sh[kPlanWaves][2];
  const int tid = threadIdx.x;
  if (tid <= kQueues) a.counters[kLine * tid] = 0;   // fetch counters: decode, then queues 0..7
  // A batch that one sweep of the work-group covers takes both passes in
  // that sweep: the first pass's scan already gives every total the second
  // pass places its items by.
  const bool one_sweep = a.num_seqs <= kPlanThreads;

  // Pass 1: sequence info, decode pairs, partial-row bases, queue sizes,
  // estimated prefill and decode costs.
  int carry[2 + kPartClasses + kQueues] = {0};
  float cost_p = 0.f, cost_d = 0.f;
  for (int base = 0; base < a.num_seqs; base += kPlanThreads) {
    const int b = base + tid;
    const SeqCounts c = seq_counts(a, b);
    if (c.ntiles > 0) {   // key tiles per item ~ (past + mid-tile row) / 64, rounded up
      const float past = (float)(c.L - c.q_len);
      float keys = past + 0.5f * (c.q_len + a.tokens_per_tile);
      if (a.window > 0) keys = fminf(keys, (float)a.window + (float)a.tokens_per_tile);
      cost_p += (float)c.ntiles * a.num_kv_heads * (keys / kPrefillKeys + 0.5f);
    } else if (c.q_len > 0) {
      cost_d += (float)(c.L - (c.s0 << a.split_shift)) * a.num_kv_heads;
    }
    // Decode pairs: every full split first (pass 1), then the
    // shorter last splits (pass 2), longest first, so the tail of the
    // decode work is made of the shortest items.
    const int has_part = (c.L & (a.split_keys - 1)) != 0 && c.nsplit > 0;
    const int pcls = part_class(c.L, a.split_shift);
    const int nfull = max(0, c.nsplit - has_part - c.s0);   // live full splits: s0 ..
    constexpr int NV = 2 + kPartClasses + kQueues;
    int v[NV], tot[NV];
    v[0] = nfull;
    v[1] = c.prows;
#pragma unroll
    for (int k = 0; k < kPartClasses; ++k) v[2 + k] = has_part && pcls == k;
#pragma unroll
    for (int x = 0; x < kQueues; ++x)
      v[2 + kPartClasses + x] = c.ntiles * heads_in_queue(b, a.num_kv_heads, x);
    block_scan<NV>(v, tot, lds);
    if (b < a.num_seqs) {
      a.seqinfo[b] = SeqInfo{c.cu0, c.q_len, c.L, carry[1] + v[1]};
      const int off = carry[0] + v[0];
      for (int s = 0; s < nfull; ++s) a.dec_items[off + s] = make_int2(b, c.s0 + s);
    }
    if (one_sweep) {
      int qpos[kQueues], run = 0;
#pragma unroll
      for (int x = 0; x < kQueues; ++x) {
        qpos[x] = run + v[2 + kPartClasses + x];
        run += tot[2 + kPartClasses + x];
      }
      int part_at = tot[0];   // after every full split: longer classes first
#pragma unroll
      for (int k = kPartClasses - 1; k >= 0; --k)
        if (k > pcls) part_at += tot[2 + k];
#pragma unroll
      for (int k = 0; k < kPartClasses; ++k)
        if (k == pcls) part_at += v[2 + k];
      emit_second_pass(a, b, c, has_part, part_at, qpos);
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) carry[k] += tot[k];
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    cost_p += __shfl_xor(cost_p, o);
    cost_d += __shfl_xor(cost_d, o);
  }
  if ((tid & 63) == 0) {
    cost_sh[tid >> 6][0] = cost_p;
    cost_sh[tid >> 6][1] = cost_d;
  }
  __syncthreads();
  if (tid == 0) {
    float sp = 0.f, sd = 0.f;
    for (int w = 0; w < kPlanWaves; ++w) {
      sp += cost_sh[w][0];
      sd += cost_sh[w][1];
    }
    const float wp = sp * kPrefillStepCost, wd = sd;
    int first = a.num_workers;
    if (wd > 0.f) first = (int)(a.num_workers * (wp / (wp + wd)) + 0.5f);
    if (wp > 0.f && first < 1) first = 1;
    a.counters[kPrefillFirst] = min(first, a.num_workers);
    int pairs = carry[0];
    for (int k = kPartClasses - 1; k >= 0; --k) {
      part_start[k] = pairs;
      pairs += carry[2 + k];
    }
    a.counters[kNumDecPairs] = pairs;
    int run = 0;
    for (int x = 0; x < kQueues; ++x) {
      a.counters[kQueueLen + x] = carry[2 + kPartClasses + x];
      a.counters[kQueueStart + x] = run;
      qstart[x] = run;
      run += carry[2 + kPartClasses + x];
    }
  }
  if (one_sweep) return;
  __syncthreads();

  // Pass 2 (batches of more than one sweep): the partial last decode splits
  // after all full ones; prefill items.
  constexpr int NV2 = kQueues + kPartClasses;
  int qcarry[NV2] = {0};
  for (int base = 0; base < a.num_seqs; base += kPlanThreads) {
    const int b = base + tid;
    const SeqCounts c = seq_counts(a, b);
    const int has_part = (c.L & (a.split_keys - 1)) != 0 && c.nsplit > 0;
    const int pcls = part_class(c.L, a.split_shift);
    int v[NV2], tot[NV2];
#pragma unroll
    for (int x = 0; x < kQueues; ++x) v[x] = c.ntiles * heads_in_queue(b, a.num_kv_heads, x);
#pragma unroll
    for (int k = 0; k < kPartClasses; ++k) v[kQueues + k] = has_part && pcls == k;
    block_scan<NV2>(v, tot, lds);
    int qpos[kQueues];
#pragma unroll
    for (int x = 0; x < kQueues; ++x) qpos[x] = qstart[x] + qcarry[x] + v[x];
    int part_at = 0;
#pragma unroll
    for (int k = 0; k < kPartClasses; ++k)
      if (k == pcls) part_at = part_start[k] + qcarry[kQueues + k] + v[kQueues + k];
    emit_second_pass(a, b, c, has_part, part_at, qpos);
#pragma unroll
    for (int x = 0; x < NV2; ++x) qcarry[x] += tot[x];
  }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace pa
