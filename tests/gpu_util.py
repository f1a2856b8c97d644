"""GPU-side test helpers: device inputs through the C ABI and oracle checks.

Inputs come from the seeded generator (paged_kv_cache_pa_amd.workloads);
the oracle gets the generator's own values (never anything the HIP path
produced) and runs its own scatter.
"""
import numpy as np
import torch

import oracle
import paged_kv_cache_pa_amd as pa
from paged_kv_cache_pa_amd import workloads as W
from pa_testutil import oracle_caches, oracle_caches_for, to_np64

TOL = {"f16": 2e-3, "bf16": 1.6e-2}
NAN_BITS = 0x7FC1   # stored bits that are a quiet NaN in both fp16 (exponent 31) and bf16 (exponent 255)


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X; run with -m 'not gpu' on the CPU")


def nan_cache(wl):
    shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_size)
    t = torch.empty(shape, dtype=torch.int16, device="cuda")
    t.fill_(NAN_BITS)
    return t.view(W.torch_dtype(wl))


def device_inputs(wl, backend="numpy", fill="nan"):
    """Values, metadata and NaN/zero-filled caches on the GPU; every KV
    position (history and new tokens) is written by pa_scatter_kv."""
    require_gpu()
    vals = W.make_values(wl, device="cuda" if backend == "torch" else "cpu", backend=backend)
    vals = {k: v.cuda() for k, v in vals.items()}
    if fill == "nan":
        kc, vc = nan_cache(wl), nan_cache(wl)
    else:
        shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_size)
        kc = torch.zeros(shape, dtype=W.torch_dtype(wl), device="cuda")
        vc = torch.zeros_like(kc)
    d = dict(vals)
    d["kc"], d["vc"] = kc, vc
    d["slots_all"] = torch.from_numpy(wl.kv_slots).cuda()
    d["slots_new"] = torch.from_numpy(wl.slot_mapping.astype(np.int32)).cuda()
    d["cu"] = torch.from_numpy(wl.cu_seqlens_q).cuda()
    d["lens"] = torch.from_numpy(wl.seqlens_kv.astype(np.int32)).cuda()
    d["table"] = torch.from_numpy(wl.block_table.astype(np.int32)).cuda()
    pa.pa_scatter_kv(d["k_all"], d["v_all"], d["slots_all"], kc, vc)
    return d


def run_attention(wl, d, **kw):
    out = pa.pa_attention(d["q"], d["cu"], d["lens"], d["table"], d["kc"], d["vc"], wl.scale,
                          wl.num_heads, wl.num_kv_heads, **kw)
    torch.cuda.synchronize()
    return out


def oracle_full(wl, d, **opts):
    """Oracle output for the whole (small) workload from the generator's
    values (``opts``: softcap, local_window_size)."""
    q = to_np64(d["q"])
    kc, vc = oracle_caches(wl, to_np64(d["k_all"]), to_np64(d["v_all"]))
    return oracle.attention(q, wl.cu_seqlens_q, wl.seqlens_kv, wl.block_table, kc, vc, wl.scale,
                            wl.num_heads, wl.num_kv_heads, wl.block_size, **opts)


def oracle_rows(wl, d, picks, **opts):
    """Oracle outputs for selected (sequence, new-row) pairs of a large
    workload.  Row i of sequence b equals a q_len=1 query whose total KV
    length is past_b + i + 1 over the same block-table row (incremental
    decoding, pinned on the oracle), so each pick is its own one-token
    sequence.  Returns float64 [len(picks), Hq, D]."""
    seqs = sorted({b for b, _ in picks})
    kv_cu = wl.kv_cu
    k_rows = lambda b: to_np64(d["k_all"][kv_cu[b]:kv_cu[b + 1]])  # noqa: E731
    v_rows = lambda b: to_np64(d["v_all"][kv_cu[b]:kv_cu[b + 1]])  # noqa: E731
    kc, vc = oracle_caches_for(wl, seqs, k_rows, v_rows)
    cu = wl.cu_seqlens_q
    toks = np.array([cu[b] + i for b, i in picks])
    q = to_np64(d["q"][torch.from_numpy(toks).cuda()])
    past = wl.seqlens_kv - wl.q_lens
    lens = np.array([past[b] + i + 1 for b, i in picks], dtype=np.int32)
    table = wl.block_table[[b for b, _ in picks]]
    return oracle.attention(q, np.arange(len(picks) + 1, dtype=np.int32), lens, table, kc, vc,
                            wl.scale, wl.num_heads, wl.num_kv_heads, wl.block_size,
                            **opts), toks


def max_err(gpu_out, ref):
    return float(np.abs(to_np64(gpu_out) - ref).max())


# ---------------------------------------------------------------- fp8 caches

FP8_NAN = 0x7F   # an e4m3 NaN code: unused slots of fp8 caches


def device_inputs_fp8(wl, backend="numpy"):
    """device_inputs with fp8 (e4m3) caches filled with NaN codes and
    seeded per-channel scales; every KV position is written by
    pa_scatter_kv_fp8."""
    require_gpu()
    vals = W.make_values(wl, device="cuda" if backend == "torch" else "cpu", backend=backend)
    d = {k: v.cuda() for k, v in vals.items()}
    shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_size)
    d["kc"] = torch.full(shape, FP8_NAN, dtype=torch.uint8, device="cuda")
    d["vc"] = torch.full(shape, FP8_NAN, dtype=torch.uint8, device="cuda")
    ks, vs = W.fp8_scales(wl)
    d["ks_np"], d["vs_np"] = ks, vs
    d["ks"], d["vs"] = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
    d["slots_all"] = torch.from_numpy(wl.kv_slots).cuda()
    d["cu"] = torch.from_numpy(wl.cu_seqlens_q).cuda()
    d["lens"] = torch.from_numpy(wl.seqlens_kv.astype(np.int32)).cuda()
    d["table"] = torch.from_numpy(wl.block_table.astype(np.int32)).cuda()
    pa.pa_scatter_kv_fp8(d["k_all"], d["v_all"], d["slots_all"], d["ks"], d["vs"], d["kc"],
                         d["vc"])
    return d


def run_attention_fp8(wl, d, max_q_len=None, **kw):
    mq = int(wl.q_lens.max()) if max_q_len is None else max_q_len
    out = pa.pa_attention_fp8(d["q"], d["cu"], d["lens"], d["table"], d["kc"], d["vc"], d["ks"],
                              d["vs"], wl.scale, wl.num_heads, wl.num_kv_heads, mq, **kw)
    torch.cuda.synchronize()
    return out


def _to_f32(t):
    return t.float().cpu().numpy()


def oracle_codes_fp8(wl, d):
    """Oracle-side code caches [NB, bs, Hk, D] (NaN codes elsewhere) from the
    oracle's own quantizing scatter of the generator's values."""
    from oracle import kv_fp8
    shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_size)
    kc = np.full(shape, FP8_NAN, np.uint8)
    vc = np.full(shape, FP8_NAN, np.uint8)
    kv_fp8.scatter_kv_fp8(_to_f32(d["k_all"]), _to_f32(d["v_all"]), wl.kv_slots, d["ks_np"],
                          d["vs_np"], kc, vc, wl.block_size)
    return kc, vc


def oracle_codes_fp8_for(wl, d, seqs):
    """Dict-of-blocks oracle code caches holding the blocks of ``seqs``."""
    from oracle import kv_fp8
    shape = (wl.block_size, wl.num_kv_heads, wl.head_size)
    kc, vc = {}, {}
    kv_cu = wl.kv_cu
    for b in seqs:
        n = int(wl.seqlens_kv[b])
        nb = -(-n // wl.block_size)
        for blk in wl.block_table[b, :nb]:
            kc.setdefault(int(blk), np.full(shape, FP8_NAN, np.uint8))
            vc.setdefault(int(blk), np.full(shape, FP8_NAN, np.uint8))
        lo, hi = int(kv_cu[b]), int(kv_cu[b + 1])
        kq = kv_fp8.quantize(_to_f32(d["k_all"][lo:hi]), d["ks_np"])
        vq = kv_fp8.quantize(_to_f32(d["v_all"][lo:hi]), d["vs_np"])
        for r, s in enumerate(wl.kv_slots[lo:hi]):
            s = int(s)
            kc[s // wl.block_size][s % wl.block_size] = kq[r]
            vc[s // wl.block_size][s % wl.block_size] = vq[r]
    return kc, vc


def oracle_full_fp8(wl, d, **opts):
    from oracle import kv_fp8
    kc, vc = oracle_codes_fp8(wl, d)
    return kv_fp8.attention_fp8(to_np64(d["q"]), wl.cu_seqlens_q, wl.seqlens_kv, wl.block_table,
                                kc, vc, d["ks_np"], d["vs_np"], wl.scale, wl.num_heads,
                                wl.num_kv_heads, wl.block_size, **opts)


def oracle_rows_fp8(wl, d, picks, **opts):
    """oracle_rows for fp8 caches: one-token sequences per (sequence, row)."""
    from oracle import kv_fp8
    seqs = sorted({b for b, _ in picks})
    kc, vc = oracle_codes_fp8_for(wl, d, seqs)
    cu = wl.cu_seqlens_q
    toks = np.array([cu[b] + i for b, i in picks])
    q = to_np64(d["q"][torch.from_numpy(toks).cuda()])
    past = wl.seqlens_kv - wl.q_lens
    lens = np.array([past[b] + i + 1 for b, i in picks], dtype=np.int32)
    table = wl.block_table[[b for b, _ in picks]]
    return kv_fp8.attention_fp8(q, np.arange(len(picks) + 1, dtype=np.int32), lens, table, kc, vc,
                                d["ks_np"], d["vs_np"], wl.scale, wl.num_heads, wl.num_kv_heads,
                                wl.block_size, **opts), toks
