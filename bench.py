#!/usr/bin/env python3
"""Benchmark of the paged-KV-cache attention hot path on one MI355X.

One step = pa_scatter_kv of the step's new K/V rows + pa_attention over the
whole continuous batch, on the large mixed workload (16 prefill chunks of
512 tokens + 240 decodes with 1k-32k contexts, 64/8 heads, D 128, block 16,
bf16).  Inputs are resident in HBM before the timed region.  The line also
carries the pure-decode and chunked-prefill workloads' figures, the
roofline of the dominant kernel, the fp64 oracle timed on host cores on a
sample of the headline batch (cpu_baseline), and per_config: every other
configuration's step latency and tokens/s with the oracle's attention and
scatter times on the host and the max abs error of the timed GPU output.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixed|decode|prefill]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_PEAK = 2.5e15         # FLOP/s, dense fp16/bf16 matrix cores
ES = 2                     # bytes per fp16/bf16 element
TOL = {"f16": 2e-3, "bf16": 1.6e-2}   # attention bars: max abs error on U(-1,1) inputs
WORKLOADS = {"tiny": 1, "small": 2, "decode": 3, "prefill": 4, "mixed": 5}


# ------------------------------------------------------------- accounting
def attention_work(wl, sel=None, kv_es=ES):
    """Algorithmic bytes and FLOPs of pa_attention over the sequences in
    ``sel``: every visible K/V element once (kv_es bytes each: 2, or 1 for
    fp8 caches, whose per-channel scales are added), Q, O, block ids and
    length metadata; FLOPs = 4*D per visible (query row, key, head)."""
    q = wl.q_lens.astype(np.int64)
    L = wl.seqlens_kv.astype(np.int64)
    if sel is None:
        sel = np.ones(len(q), dtype=bool)
    q, L = q[sel], L[sel]
    past = L - q
    D, hq, hk, bs = wl.head_size, wl.num_heads, wl.num_kv_heads, wl.block_size
    kv = int((L * hk * D * 2 * kv_es).sum()) + (2 * hk * D * 4 if kv_es == 1 else 0)
    qo = int(2 * q.sum() * hq * D * ES)
    ids = int((-(-L // bs)).sum() * 4 + (2 * len(q) + 1) * 4)
    flops = int(4 * D * hq * (q * past + q * (q + 1) // 2).sum())
    return kv + qo + ids, flops


def scatter_work(wl, kv_es=ES):
    T = wl.num_tokens
    return 2 * T * wl.num_kv_heads * wl.head_size * (ES + kv_es) + 4 * T


def roofline_time(nbytes, flops):
    return max(nbytes / HBM_PEAK, flops / MFMA_PEAK)


# ------------------------------------------------------------- GPU side
def setup(wl, torch, pa, W, fp8=False, opts=None):
    vals = W.make_values(wl, device="cuda", backend="torch")
    dt = W.torch_dtype(wl)
    shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_size)
    kc = torch.zeros(shape, dtype=torch.uint8 if fp8 else dt, device="cuda")
    vc = torch.zeros_like(kc)
    slots_all = torch.from_numpy(wl.kv_slots).cuda()
    extra = {}
    if fp8:
        ks, vs = W.fp8_scales(wl)
        extra = dict(fp8=True, ks=torch.from_numpy(ks).cuda(), vs=torch.from_numpy(vs).cuda(),
                     max_q_len=int(wl.q_lens.max()))
        pa.pa_scatter_kv_fp8(vals["k_all"], vals["v_all"], slots_all, extra["ks"], extra["vs"],
                             kc, vc)
    else:
        pa.pa_scatter_kv(vals["k_all"], vals["v_all"], slots_all, kc, vc)
    new_rows = torch.from_numpy(wl.new_rows).cuda()
    st = dict(q=vals["q"], k_new=vals["k_all"][new_rows].contiguous(),
              v_new=vals["v_all"][new_rows].contiguous(), kc=kc, vc=vc,
              slots=torch.from_numpy(wl.slot_mapping.astype(np.int32)).cuda(),
              cu=torch.from_numpy(wl.cu_seqlens_q).cuda(),
              lens=torch.from_numpy(wl.seqlens_kv.astype(np.int32)).cuda(),
              table=torch.from_numpy(wl.block_table.astype(np.int32)).cuda(), vals=vals,
              opts=dict(opts or {}), **extra)
    st["out"] = torch.empty((wl.num_tokens, wl.num_heads, wl.head_size), dtype=dt, device="cuda")
    n = pa.pa_attention_workspace_size(wl.num_seqs, wl.num_tokens, wl.max_blocks_per_seq,
                                       wl.num_heads, wl.num_kv_heads, wl.head_size,
                                       wl.block_size)
    st["ws"] = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    return st


def step(wl, st, pa):
    if st.get("fp8"):
        pa.pa_scatter_kv_fp8(st["k_new"], st["v_new"], st["slots"], st["ks"], st["vs"], st["kc"],
                             st["vc"])
        pa.pa_attention_fp8(st["q"], st["cu"], st["lens"], st["table"], st["kc"], st["vc"],
                            st["ks"], st["vs"], wl.scale, wl.num_heads, wl.num_kv_heads,
                            st["max_q_len"], out=st["out"], workspace=st["ws"], **st["opts"])
        return
    pa.pa_scatter_kv(st["k_new"], st["v_new"], st["slots"], st["kc"], st["vc"])
    pa.pa_attention(st["q"], st["cu"], st["lens"], st["table"], st["kc"], st["vc"], wl.scale,
                    wl.num_heads, wl.num_kv_heads, out=st["out"], workspace=st["ws"],
                    **st["opts"])


SCRUB_BYTES = 512 << 20     # swept between separately timed reps (larger than the 256 MB MALL)


def scrub_caches(scrub, i, torch, write=False):
    """Evict every cache level: read all of `scrub` (a reduction over it), or
    with `write`, overwrite it.  A write scrub leaves a cache's worth of
    dirty lines whose write-back the next timed rep pays for (26 us on the
    pure-decode step), so the default sweep only reads."""
    if write:
        scrub.fill_(i & 255)
        return None
    return scrub.view(torch.int32).amax()


def per_rep_times(fn, reps, torch, scrub, write_scrub=False):
    """Each rep timed on its own with HIP events, after a sweep of `scrub`
    (outside the events) so that no cache level still holds the previous
    rep's data.  Median, min and p90 over the reps."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    sink = []
    for i, (a, b) in enumerate(ev):
        sink.append(scrub_caches(scrub, i, torch, write_scrub))
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return {"reps": reps, "scrub_MiB": scrub.numel() >> 20,
            "scrub": "write" if write_scrub else "read",
            "median_ms": float(np.median(t)), "min_ms": float(t[0]),
            "p90_ms": float(np.percentile(t, 90))}


def sub_batch(wl, st, sel, torch, pa):
    """Device inputs of pa_attention over the sequences in `sel` only; their
    K/V already sit in the shared, filled cache."""
    idx = np.flatnonzero(sel)
    cu = wl.cu_seqlens_q
    rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in idx]).astype(np.int64)
    ql = wl.q_lens[idx]
    q = st["q"][torch.from_numpy(rows).cuda()].contiguous()
    sub = {"q": q, "kc": st["kc"], "vc": st["vc"], "out": torch.empty_like(q),
           "cu": torch.from_numpy(np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)).cuda(),
           "lens": torch.from_numpy(wl.seqlens_kv[idx].astype(np.int32)).cuda(),
           "table": torch.from_numpy(np.ascontiguousarray(wl.block_table[idx]).astype(np.int32)).cuda()}
    n = pa.pa_attention_workspace_size(len(idx), int(ql.sum()), wl.max_blocks_per_seq, wl.num_heads,
                                       wl.num_kv_heads, wl.head_size, wl.block_size)
    sub["ws"] = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    return sub


def time_workload(wl, steps, warmup, torch, pa, W, extras=False, fp8=False, opts=None,
                  keep=False):
    """Back-to-back timing of `steps` steps (the headline figure) and the
    per-kernel averages; with `extras`, also per-rep scrubbed timing of the
    step and, for a batch that mixes both kinds, its decode-only and
    prefill-only sub-batches timed as separate pa_attention calls.  `opts`:
    attention options (softcap, local_window_size) of every call."""
    st = setup(wl, torch, pa, W, fp8=fp8, opts=opts)
    for _ in range(warmup):
        step(wl, st, pa)
    torch.cuda.synchronize()
    # Only the attention kernel is bracketed with events in the timed steps
    # (events around all four kernels add about 30 us to a 2.3 ms step); the
    # other kernels' averages come from an untimed pass afterwards.
    pa.profile_read()                       # drop anything recorded earlier
    pa.profile_select(["attention"])
    pa.profile_enable(True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step(wl, st, pa)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pa.profile_enable(False)
    kern = pa.profile_read()
    ms = e0.elapsed_time(e1) / steps
    pa.profile_select(None)
    pa.profile_enable(True)
    for _ in range(steps):
        step(wl, st, pa)
    torch.cuda.synchronize()
    pa.profile_enable(False)
    kern = {k: (kern[k] if k == "attention" else v) for k, v in pa.profile_read().items()}
    per_kernel = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in kern.items()}
    more = {}
    if keep:   # the timed run's output and the inputs it was computed from
        more["out"] = st["out"].clone()
        more["vals"] = st["vals"]
    if extras:
        scrub = torch.zeros(SCRUB_BYTES, dtype=torch.uint8, device="cuda")
        more["step_reps"] = per_rep_times(lambda: step(wl, st, pa), steps, torch, scrub)
        more["step_reps_write_scrub"] = per_rep_times(lambda: step(wl, st, pa), steps, torch,
                                                      scrub, write_scrub=True)
        if fp8:
            del scrub, st
            torch.cuda.empty_cache()
            return ms, wall / steps * 1e3, per_kernel, more
        # Both scatter entry points on this step's new tokens: slots from the
        # host-side slot_mapping, and slots derived on the GPU from the
        # block table (pa_scatter_kv_paged).
        sc_bytes = scatter_work(wl)
        scat = {}
        for name, fn in (
                ("slot_mapping", lambda: pa.pa_scatter_kv(st["k_new"], st["v_new"], st["slots"],
                                                          st["kc"], st["vc"])),
                ("paged", lambda: pa.pa_scatter_kv_paged(st["k_new"], st["v_new"], st["cu"],
                                                         st["lens"], st["table"], st["kc"],
                                                         st["vc"]))):
            fn()
            r = per_rep_times(fn, steps, torch, scrub)
            r["GBps"] = sc_bytes / (r["median_ms"] * 1e-3) / 1e9
            scat[name] = r
        scat["bytes"] = sc_bytes
        more["scatter"] = scat
        G = wl.num_heads // wl.num_kv_heads
        dec_sel = (wl.q_lens * G <= 16) & (wl.q_lens > 0)
        pf_sel = wl.q_lens * G > 16
        if dec_sel.any() and pf_sel.any():
            subs = {}
            for name, sel in (("decode_only", dec_sel), ("prefill_only", pf_sel)):
                sb = sub_batch(wl, st, sel, torch, pa)
                call = lambda sb=sb: pa.pa_attention(  # noqa: E731
                    sb["q"], sb["cu"], sb["lens"], sb["table"], sb["kc"], sb["vc"], wl.scale,
                    wl.num_heads, wl.num_kv_heads, out=sb["out"], workspace=sb["ws"],
                    **st["opts"])
                for _ in range(3):
                    call()
                r = per_rep_times(call, steps, torch, scrub)
                nbytes, flops = attention_work(wl, sel)
                t = r["median_ms"] * 1e-3
                r.update({"num_seqs": int(sel.sum()), "alg_bytes": nbytes, "alg_flops": flops,
                          "TBps": nbytes / t / 1e12, "TFLOPs": flops / t / 1e12,
                          "roofline_frac": roofline_time(nbytes, flops) / t})
                subs[name] = r
                del sb
            subs["note"] = ("the two kinds of sequence of the same batch as separate pa_attention "
                            "calls (same cache); their sum against the one mixed call shows what "
                            "running both kinds in one launch gains")
            subs["sum_of_separate_ms"] = subs["decode_only"]["median_ms"] + subs["prefill_only"]["median_ms"]
            more["sub_batches"] = subs
        # The fused step ahead of the attention on this batch's new tokens:
        # packed QKV rows split, Q and K rotated over the whole head (split
        # pairing), K/V scattered (pa_rotary_scatter_kv).  Timed last: it
        # leaves rotated K in the cache.
        T = wl.num_tokens
        packed = torch.cat([st["q"].reshape(T, -1), st["k_new"].reshape(T, -1),
                            st["v_new"].reshape(T, -1)], dim=1).contiguous()
        cos, sin = W.rope_tables(int(wl.seqlens_kv.max()), wl.head_size, wl.dtype)
        cos, sin = cos.cuda(), sin.cuda()
        q_rot = torch.empty_like(st["q"])
        fn = lambda: pa.pa_rotary_scatter_kv(  # noqa: E731
            packed, st["cu"], st["lens"], st["table"], st["kc"], st["vc"], wl.num_heads,
            wl.num_kv_heads, cos_cache=cos, sin_cache=sin, q_out=q_rot)
        fn()
        r = per_rep_times(fn, steps, torch, scrub)
        nbytes = 2 * packed.numel() * packed.element_size()   # every element read once, written once
        r.update({"bytes": nbytes, "GBps": nbytes / (r["median_ms"] * 1e-3) / 1e9,
                  "rotary_dim": wl.head_size, "pairing": "split", "input": "packed QKV"})
        more["rotary_scatter"] = r
        # The whole rotary step: that scatter writing the rotated Q and
        # pa_attention reading it back, against the scatter leaving Q alone
        # and pa_attention_rope rotating Q from the packed rows as it loads
        # it (same output bits).
        qv = packed.view(T, -1, wl.head_size)
        two = lambda: (fn(), pa.pa_attention(  # noqa: E731
            q_rot, st["cu"], st["lens"], st["table"], st["kc"], st["vc"], wl.scale, wl.num_heads,
            wl.num_kv_heads, out=st["out"], workspace=st["ws"], **st["opts"]))
        fused = lambda: (pa.pa_rotary_scatter_kv(  # noqa: E731
            packed, st["cu"], st["lens"], st["table"], st["kc"], st["vc"], wl.num_heads,
            wl.num_kv_heads, cos_cache=cos, sin_cache=sin, write_q=False), pa.pa_attention_rope(
            qv, st["cu"], st["lens"], st["table"], st["kc"], st["vc"], wl.scale, wl.num_heads,
            wl.num_kv_heads, cos_cache=cos, sin_cache=sin, out=st["out"], workspace=st["ws"],
            **st["opts"]))
        rs = {}
        for name, f in (("two_step", two), ("fused", fused)):
            f()
            rs[name] = per_rep_times(f, steps, torch, scrub)
        rs["note"] = ("pa_rotary_scatter_kv + pa_attention on its rotated Q, against the scatter "
                      "without Q + pa_attention_rope on the packed rows (Q rotated on load)")
        rs["fused_vs_two_step"] = rs["fused"]["median_ms"] / rs["two_step"]["median_ms"]
        more["rope_step"] = rs
        del packed, q_rot, qv
        del scrub
    del st
    torch.cuda.empty_cache()
    return ms, wall / steps * 1e3, per_kernel, more


def summarize(wl, ms, per_kernel, kv_es=ES):
    """Throughputs of one step and of its attention kernel (the one launch
    that runs both the prefill tiles and the split-KV decode items); kv_es 1
    for fp8 caches."""
    att_bytes, att_flops = attention_work(wl, kv_es=kv_es)
    nbytes = att_bytes + scatter_work(wl, kv_es=kv_es)
    t = ms * 1e-3
    dec_sel = (wl.q_lens * (wl.num_heads // wl.num_kv_heads) <= 16) & (wl.q_lens > 0)
    pf_sel = wl.q_lens * (wl.num_heads // wl.num_kv_heads) > 16
    r = {
        "ms_per_step": ms,
        "roofline_pct": 100.0 * roofline_time(nbytes, att_flops) / t,
        "tokens_per_s": wl.num_tokens / t,
        "alg_bytes": nbytes,
        "alg_flops": att_flops,
        "kernel_ms": {k: round(v, 5) for k, v in per_kernel.items()},
    }
    ta = per_kernel.get("attention", 0.0) * 1e-3
    if ta > 0:
        r["attention_alg_bytes"] = att_bytes
        r["attention_alg_flops"] = att_flops
        r["attention_TBps"] = att_bytes / ta / 1e12
        r["attention_TFLOPs"] = att_flops / ta / 1e12
        r["attention_roofline_frac"] = roofline_time(att_bytes, att_flops) / ta
        r["attention_bound"] = "hbm" if att_bytes / HBM_PEAK >= att_flops / MFMA_PEAK else "mfma"
        if not pf_sel.any():       # decode only: the kernel's bytes are the decode bytes
            r["decode_TBps"] = r["attention_TBps"]
            r["decode_hbm_frac"] = r["decode_TBps"] * 1e12 / HBM_PEAK
        if not dec_sel.any():      # prefill only
            r["prefill_TFLOPs"] = r["attention_TFLOPs"]
            r["prefill_mfma_frac"] = r["prefill_TFLOPs"] * 1e12 / MFMA_PEAK
    return r


def strip_comments(src):
    """C++ source without its // and /* */ comments (string and character
    literals kept as they are)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "".join(out)


def kernel_source_hash(sources=None):
    """Hash of the code the kernels are compiled from: every file under
    csrc/ except pa_api.hip (the C-ABI host code, which holds no kernel),
    with comments removed and runs of white space made one space, so that
    only a change of code marks recorded counters as stale.  ``sources``: {file name: text} in place of the
    files on disk."""
    if sources is None:
        csrc = os.path.join(ROOT, "paged_kv_cache_pa_amd", "csrc")
        sources = {f: open(os.path.join(csrc, f)).read() for f in os.listdir(csrc)}
    h = hashlib.sha256()
    for f in sorted(sources):
        if f == "pa_api.hip":
            continue
        h.update(f.encode() + b"\0" + " ".join(strip_comments(sources[f]).split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch recorded from rocprofv3 counters for this kernel
    source (profiles/traffic.json); None when absent or stale."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = rec.get(f"{workload}:{kernel}")
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def copy_bandwidth(torch, nbytes=2 << 30, reps=10):
    """Device-to-device copy of a 2 GiB buffer (read + write counted), the
    measured reference for the HBM peak on this machine."""
    src = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda")
    src.fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / t / 1e9


# ------------------------------------------------------------- CPU baseline
def cpu_baseline(wl, W, torch, budget_s=20.0, opts=None):
    """The fp64 oracle (as it stands) on a bounded sample of the workload:
    the first decode sequences and, if any, the first prefill chunks;
    reported in the metric's unit and as tokens/s.  `opts`: the attention
    options of the GPU run."""
    import oracle
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    vals = W.make_values(wl, device="cuda", backend="torch")
    kv_cu, cu = wl.kv_cu, wl.cu_seqlens_q
    dec = [int(b) for b in np.flatnonzero(wl.q_lens == 1)]
    pre = [int(b) for b in np.flatnonzero(wl.q_lens > 1)]
    picks = pre[:6] + dec[:96]      # ~10 s of fp64 oracle work on the host
    shape = (wl.block_size, wl.num_kv_heads, wl.head_size)
    kc, vc = {}, {}
    for b in picks:
        nb = -(-int(wl.seqlens_kv[b]) // wl.block_size)
        for x in wl.block_table[b, :nb]:
            kc.setdefault(int(x), np.zeros(shape))
            vc.setdefault(int(x), np.zeros(shape))
        oracle.scatter_kv(f64(vals["k_all"][kv_cu[b]:kv_cu[b + 1]]),
                          f64(vals["v_all"][kv_cu[b]:kv_cu[b + 1]]),
                          wl.kv_slots[kv_cu[b]:kv_cu[b + 1]], kc, vc, wl.block_size)
    q_parts = [f64(vals["q"][cu[b]:cu[b + 1]]) for b in picks]
    # this step's new K/V rows of the sample (the last q_len positions of each)
    new_lo = [int(kv_cu[b + 1] - wl.q_lens[b]) for b in picks]
    new_k = [f64(vals["k_all"][lo:kv_cu[b + 1]]) for lo, b in zip(new_lo, picks)]
    new_v = [f64(vals["v_all"][lo:kv_cu[b + 1]]) for lo, b in zip(new_lo, picks)]
    new_slots = [wl.kv_slots[lo:kv_cu[b + 1]] for lo, b in zip(new_lo, picks)]
    del vals
    torch.cuda.empty_cache()
    q_lens = np.array([wl.q_lens[b] for b in picks], dtype=np.int32)
    sub_cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    sub_lens = np.array([wl.seqlens_kv[b] for b in picks], dtype=np.int32)
    sub_table = wl.block_table[picks]
    q = np.concatenate(q_parts, axis=0)
    t0 = time.perf_counter()
    oracle.scatter_kv(np.concatenate(new_k), np.concatenate(new_v), np.concatenate(new_slots),
                      kc, vc, wl.block_size)
    t_scatter = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.attention(q, sub_cu, sub_lens, sub_table, kc, vc, wl.scale, wl.num_heads,
                     wl.num_kv_heads, wl.block_size, **(opts or {}))
    t = time.perf_counter() - t0
    sel = np.zeros(wl.num_seqs, dtype=bool)
    sel[picks] = True
    nbytes, flops = attention_work(wl, sel)
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        blas = None
    cores = len(os.sched_getaffinity(0))
    return {"value": 100.0 * roofline_time(nbytes, flops) / t, "unit": "% of MI355X roofline",
            "tokens_per_s": float(q_lens.sum()) / t, "seconds": t,
            "scatter_seconds": t_scatter,
            "scatter_tokens_per_s": float(q_lens.sum()) / max(t_scatter, 1e-9),
            "cores": int(blas or cores), "host_cpus": os.cpu_count(), "affinity_cpus": cores,
            "kind": "oracle",
            "sample": f"fp64 NumPy oracle (attention timed apart from the scatter of the sample's "
                      f"new tokens) on {len(pre[:6])} prefill chunk(s) "
                      f"of 512 tokens + {len(dec[:96])} decode sequences of the same workload "
                      f"({int(q_lens.sum())} query tokens)"}


# ------------------------------------------------------------- per config
def _host_rows(t):
    """GPU fp16/bf16 rows -> host float32 (exact), kept as float32 to halve
    host memory; converted to float64 per sequence."""
    return t.float().cpu().numpy()


def oracle_check(wl, vals, out, threads, opts=None):
    """The fp64 oracle over every sequence of a workload, in three phases:
    each sequence's past rows are scattered into a dict-of-blocks cache of
    its own (untimed); the step's new rows of every sequence are scattered
    (timed, one thread: the scatter); the attention of every sequence's new
    rows is computed one sequence at a time on `threads` host threads with
    BLAS held to one thread each (timed: the attention).  Returns both wall
    times, the thread counts and the max abs error of `out` (the GPU output
    of the timed run)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    k_all, v_all = _host_rows(vals["k_all"]), _host_rows(vals["v_all"])
    qh = vals["q"].float().cpu().numpy().astype(np.float64)
    oh = out.float().cpu().numpy().astype(np.float64)
    cu, kv_cu = wl.cu_seqlens_q, wl.kv_cu
    shape = (wl.block_size, wl.num_kv_heads, wl.head_size)
    seqs = [b for b in range(wl.num_seqs) if cu[b + 1] > cu[b]]
    caches = {}

    def build(b):        # float32 holds the fp16/bf16 values exactly
        lo, nl = int(kv_cu[b]), int(kv_cu[b + 1] - wl.q_lens[b])
        kc, vc = {}, {}
        for x in wl.block_table[b, :-(-int(wl.seqlens_kv[b]) // wl.block_size)]:
            kc.setdefault(int(x), np.zeros(shape, np.float32))
            vc.setdefault(int(x), np.zeros(shape, np.float32))
        oracle.scatter_kv(k_all[lo:nl], v_all[lo:nl], wl.kv_slots[lo:nl], kc, vc, wl.block_size)
        caches[b] = (kc, vc)

    def attend(b):
        kc, vc = caches[b]
        ql = int(cu[b + 1] - cu[b])
        ref = oracle.attention(qh[cu[b]:cu[b + 1]], np.array([0, ql], np.int32),
                               wl.seqlens_kv[b:b + 1], wl.block_table[b:b + 1], kc, vc, wl.scale,
                               wl.num_heads, wl.num_kv_heads, wl.block_size, **(opts or {}))
        return float(np.abs(oh[cu[b]:cu[b + 1]] - ref).max())

    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except ImportError:
        import contextlib
        limit = contextlib.nullcontext()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(build, seqs))
    t0 = time.perf_counter()
    for b in seqs:
        nl, hi = int(kv_cu[b + 1] - wl.q_lens[b]), int(kv_cu[b + 1])
        oracle.scatter_kv(k_all[nl:hi].astype(np.float64), v_all[nl:hi].astype(np.float64),
                          wl.kv_slots[nl:hi], caches[b][0], caches[b][1], wl.block_size)
    t_scatter = time.perf_counter() - t0
    order = sorted(seqs, key=lambda b: -int(wl.q_lens[b]) * int(wl.seqlens_kv[b])
                   - int(wl.seqlens_kv[b]))
    t0 = time.perf_counter()
    with limit, ThreadPoolExecutor(threads) as ex:
        errs = list(ex.map(attend, order))
    t_att = time.perf_counter() - t0
    return {"attention_s": t_att, "attention_threads": threads, "scatter_s": t_scatter,
            "scatter_threads": 1, "max_abs_err": max(errs) if errs else 0.0}


def per_config(steps, warmup, torch, pa, W):
    """Every configuration apart from the headline one: GPU step latency
    (pa_scatter_kv of the step's new tokens + pa_attention, back to back
    after warm-up) and tokens/s, and the fp64 oracle on the host cores
    (attention and scatter timed apart) with the max abs error of the GPU
    output of the timed run against it.  The small configuration is the
    84-case matrix: latency over the cases, the worst error."""
    threads = min(16, len(os.sched_getaffinity(0)))
    res = {}
    for name, idx in (("tiny", 1), ("decode", 3), ("prefill", 4)):
        wl = W.by_index(idx)
        ms, _, pk, more = time_workload(wl, steps, warmup, torch, pa, W, keep=True)
        r = {"workload": wl.name, "dtype": wl.dtype, "step_us": ms * 1e3,
             "attention_us": pk.get("attention", 0.0) * 1e3,
             "tokens_per_s": wl.num_tokens / (ms * 1e-3)}
        r["oracle"] = oracle_check(wl, more["vals"], more["out"], threads)
        r["oracle"]["tolerance"] = TOL[wl.dtype]
        res[name] = r
        del more
        torch.cuda.empty_cache()
    lat, toks, worst, o_att, o_sc = [], 0, 0.0, 0.0, 0.0
    for n, (qs, ls, hq, hk) in enumerate(W.small_cases()):
        wl = W.small(qs, ls, hq, hk, seed=2000 + n)
        ms, _, pk, more = time_workload(wl, steps, warmup, torch, pa, W, keep=True)
        lat.append(ms * 1e3)
        toks += wl.num_tokens
        o = oracle_check(wl, more["vals"], more["out"], 1)
        worst = max(worst, o["max_abs_err"])
        o_att += o["attention_s"]
        o_sc += o["scatter_s"]
    res["small"] = {"workload": f"small matrix: {len(lat)} cases (q_len {{1,4,16}}, total "
                                f"{{32,64}}, MHA 8/8 and GQA 8/2, D 64, bs 256, fp16)",
                    "dtype": "f16", "step_us_median": float(np.median(lat)),
                    "step_us_min": float(min(lat)), "step_us_max": float(max(lat)),
                    "tokens_per_s": toks / (sum(lat) * 1e-6),
                    "oracle": {"attention_s": o_att, "attention_threads": 1,
                               "scatter_s": o_sc, "scatter_threads": 1, "max_abs_err": worst,
                               "tolerance": TOL["f16"], "note": "summed over the 84 cases"}}
    return res


# ------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixed", choices=sorted(WORKLOADS))
    ap.add_argument("--no-extra", action="store_true", help="skip the decode/prefill figures")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fp8", action="store_true",
                    help="fp8 (e4m3) caches (pa_scatter_kv_fp8 + pa_attention_fp8); "
                         "decode-shaped workloads only")
    ap.add_argument("--softcap", type=float, default=0.0,
                    help="score soft cap c of every attention call (0: off)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window (local_window_size) of every attention call (0: off)")
    ap.add_argument("--copy-only", action="store_true",
                    help="only the 2 GiB copy (reference for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the paged attention hot path is measured on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_pa_amd as pa
    from paged_kv_cache_pa_amd import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pa._lib.lib()           # fail loudly when the HIP library is missing
    if args.copy_only:
        print(json.dumps({"copy_GBps": copy_bandwidth(torch), "bytes": 2 * (2 << 30)}))
        return
    copy_gbps = copy_bandwidth(torch)

    wl = W.by_index(WORKLOADS[args.workload])
    if args.fp8 and (wl.q_lens * (wl.num_heads // wl.num_kv_heads)).max() > 16:
        print("--fp8 needs a decode-shaped workload (every q_len * G <= 16)", file=sys.stderr)
        sys.exit(2)
    opts = {}
    if args.softcap > 0:
        opts["softcap"] = args.softcap
    if args.window > 0:
        opts["local_window_size"] = args.window
    ms, wall_ms, per_kernel, more = time_workload(wl, args.steps, args.warmup, torch, pa, W,
                                                  extras=not args.no_extra, fp8=args.fp8,
                                                  opts=opts)
    head = summarize(wl, ms, per_kernel, kv_es=1 if args.fp8 else ES)
    if head.get("attention_bound") == "mfma":
        ach = head["attention_TFLOPs"]
        roof = {"bound": "mfma", "kernel": "attention_kernel", "achieved": ach, "peak": 2500.0,
                "unit": "TFLOP/s", "frac": ach / 2500.0,
                "alg_flops_per_launch": head["attention_alg_flops"]}
    else:
        ach = head.get("attention_TBps", 0.0) * 1e3
        roof = {"bound": "hbm", "kernel": "attention_kernel", "achieved": ach, "peak": 8000.0,
                "unit": "GB/s", "frac": ach / 8000.0,
                "alg_bytes_per_launch": head.get("attention_alg_bytes")}
    if args.fp8:
        roof["kernel"] = "attention_kernel_fp8"
    roof["avg_launch_ms"] = per_kernel.get("attention", 0.0)
    roof["traffic"] = measured_traffic(roof["kernel"], args.workload + ("_fp8" if args.fp8 else ""))

    extra = {}
    if not args.no_extra and args.workload == "mixed":
        for name in ("decode", "prefill"):
            w2 = W.by_index(WORKLOADS[name])
            m2, _, k2, more2 = time_workload(w2, max(5, args.steps // 2), 3, torch, pa, W,
                                             extras=True)
            extra[name] = summarize(w2, m2, k2)
            extra[name]["workload"] = w2.name
            extra[name]["step_reps"] = more2.get("step_reps")
            extra[name]["step_reps_write_scrub"] = more2.get("step_reps_write_scrub")
        # The pure-decode workload again on fp8 (e4m3) caches with per-channel
        # scales (pa_scatter_kv_fp8 + pa_attention_fp8): half the cache bytes.
        w2 = W.by_index(WORKLOADS["decode"])
        m2, _, k2, more2 = time_workload(w2, max(5, args.steps // 2), 3, torch, pa, W,
                                         extras=True, fp8=True)
        e = summarize(w2, m2, k2, kv_es=1)
        e["workload"] = w2.name + ", fp8 e4m3 caches with per-channel scales"
        e["step_reps"] = more2.get("step_reps")
        e["step_reps_write_scrub"] = more2.get("step_reps_write_scrub")
        a16 = extra["decode"]["kernel_ms"].get("attention", 0.0)
        a8 = e["kernel_ms"].get("attention", 0.0)
        e["attention_speedup_vs_16bit_cache"] = a16 / a8 if a8 > 0 else None
        extra["decode_fp8"] = e
        # The headline batch again with the score options on: attention time
        # against the plain call (a window also cuts the keys read).
        if not opts:
            a0 = head["kernel_ms"].get("attention", 0.0)
            o = {}
            for name, kw in (("softcap_50", dict(softcap=50.0)),
                             ("window_4096", dict(local_window_size=4096)),
                             ("softcap_50_window_4096", dict(softcap=50.0,
                                                             local_window_size=4096))):
                m2, _, k2, _ = time_workload(wl, max(5, args.steps // 2), 3, torch, pa, W,
                                             opts=kw)
                a2 = k2.get("attention", 0.0)
                o[name] = {"ms_per_step": m2, "attention_ms": a2,
                           "attention_time_vs_plain": a2 / a0 if a0 > 0 else None}
            extra["options"] = o

    line = {
        "metric": "paged-attn decode HBM TB/s + prefill TFLOP/s, % of MI355X roofline",
        "value": head["roofline_pct"],
        "unit": "% of MI355X roofline (max(bytes/8TB/s, flops/2.5PF) / step time)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "wall_ms_per_step": wall_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "num_seqs": wl.num_seqs, "num_tokens": wl.num_tokens,
                   "step": "pa_scatter_kv(new tokens) + pa_attention(whole batch)",
                   "parallelism": "single GPU", **opts},
        "tokens_per_s": head["tokens_per_s"],
        "attention_TBps": head.get("attention_TBps"),
        "attention_TFLOPs": head.get("attention_TFLOPs"),
        "decode_TBps": head.get("decode_TBps") or extra.get("decode", {}).get("decode_TBps"),
        "prefill_TFLOPs": (head.get("prefill_TFLOPs")
                           or extra.get("prefill", {}).get("prefill_TFLOPs")),
        "kernel_ms": head["kernel_ms"],
        "copy_GBps": copy_gbps,
        "roofline": roof,
        "step_reps": more.get("step_reps"),
        "step_reps_write_scrub": more.get("step_reps_write_scrub"),
        "sub_batches": more.get("sub_batches"),
        "scatter": more.get("scatter"),
        "rotary_scatter": more.get("rotary_scatter"),
        "rope_step": more.get("rope_step"),
        "extra": extra,
    }
    if not args.no_extra and args.workload == "mixed" and not opts:
        line["per_config"] = per_config(max(5, args.steps // 2), 3, torch, pa, W)
    if opts.get("local_window_size"):
        line["note"] = ("algorithmic bytes and flops count the plain causal work; the window "
                        "reads and computes less, so the rates above overstate it")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, W, torch, opts=opts)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
