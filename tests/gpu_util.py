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
NAN_BITS = 0x7E01   # a quiet-NaN payload in both fp16 and bf16 as stored bits


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


def oracle_full(wl, d):
    """Oracle output for the whole (small) workload from the generator's
    values."""
    q = to_np64(d["q"])
    kc, vc = oracle_caches(wl, to_np64(d["k_all"]), to_np64(d["v_all"]))
    return oracle.attention(q, wl.cu_seqlens_q, wl.seqlens_kv, wl.block_table, kc, vc, wl.scale,
                            wl.num_heads, wl.num_kv_heads, wl.block_size)


def oracle_rows(wl, d, picks):
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
                            wl.scale, wl.num_heads, wl.num_kv_heads, wl.block_size), toks


def max_err(gpu_out, ref):
    return float(np.abs(to_np64(gpu_out) - ref).max())
