"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bars: scatter and every cache byte bit-exact; attention max abs error
<= 2e-3 (fp16) / 1.6e-2 (bf16) on U(-1,1) inputs (and the N(0,1) decode
workload); closed-form cases exact.  Unused cache slots hold NaN in every
test, so any read of them shows up as a non-finite output.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_pa_amd as pa
from paged_kv_cache_pa_amd import workloads as W
from gpu_util import (NAN_BITS, TOL, device_inputs, max_err, nan_cache, oracle_full, oracle_rows,
                      require_gpu, run_attention)
from pa_testutil import embed_flex_example, load_golden, oracle_caches, to_np64

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# ---------------------------------------------------------------- scatter

@pytest.mark.parametrize("make", [W.tiny, lambda: W.small((16, 4), (64, 32), 8, 2),
                                  lambda: W.custom([3, 1, 7], [40, 1, 300], 8, 2, 128, 32,
                                                   dtype="bf16")])
def test_scatter_bit_exact_small(make):
    wl = make()
    _log(f"scatter: {wl.name}")
    d = device_inputs(wl)
    kb, vb = _bits(d["k_all"]), _bits(d["v_all"])
    shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_size)
    kref = np.full(shape, NAN_BITS, dtype=np.uint16)
    vref = np.full(shape, NAN_BITS, dtype=np.uint16)
    oracle.scatter_kv(kb, vb, wl.kv_slots, kref, vref, wl.block_size)
    assert np.array_equal(_bits(d["kc"]), kref)
    assert np.array_equal(_bits(d["vc"]), vref)
    # The new-token scatter alone rewrites the same bytes, and negative
    # slots write nothing.
    slots = d["slots_new"].clone()
    slots[0] = -1
    knew = torch.zeros_like(d["k_all"][: wl.num_tokens])
    pa.pa_scatter_kv(knew, knew, slots, d["kc"], d["vc"])
    torch.cuda.synchronize()
    s = wl.slot_mapping.astype(np.int64)
    flat_k = _bits(d["kc"]).reshape(-1, wl.num_kv_heads * wl.head_size)
    assert np.array_equal(flat_k[s[0]], kref.reshape(flat_k.shape)[s[0]])
    assert (flat_k[s[1:]] == 0).all()


@pytest.mark.parametrize("idx", [3, 4, 5])
def test_scatter_bit_exact_large(idx):
    """Multi-GB pools (element offsets beyond 2^31): sampled sequences'
    blocks match the oracle's scatter bit for bit, untouched blocks keep the
    NaN sentinel."""
    wl = W.by_index(idx)
    _log(f"scatter: {wl.name}")
    d = device_inputs(wl, backend="torch")
    rng = np.random.default_rng(idx)
    seqs = list(rng.choice(wl.num_seqs, size=4, replace=False))
    seqs.append(int(np.argmax(wl.block_table.max(axis=1))))   # the highest block id in use
    kv_cu = wl.kv_cu
    shape = (wl.block_size, wl.num_kv_heads, wl.head_size)
    for b in seqs:
        kb = _bits(d["k_all"][kv_cu[b]:kv_cu[b + 1]])
        vb = _bits(d["v_all"][kv_cu[b]:kv_cu[b + 1]])
        nb = -(-int(wl.seqlens_kv[b]) // wl.block_size)
        blocks = [int(x) for x in wl.block_table[b, :nb]]
        kref = {x: np.full(shape, NAN_BITS, dtype=np.uint16) for x in blocks}
        vref = {x: np.full(shape, NAN_BITS, dtype=np.uint16) for x in blocks}
        oracle.scatter_kv(kb, vb, wl.kv_slots[kv_cu[b]:kv_cu[b + 1]], kref, vref, wl.block_size)
        for x in blocks:
            assert np.array_equal(_bits(d["kc"][x]), kref[x]), (b, x)
            assert np.array_equal(_bits(d["vc"][x]), vref[x]), (b, x)
    used = np.zeros(wl.num_blocks, dtype=bool)
    for b in range(wl.num_seqs):
        used[wl.block_table[b, : -(-int(wl.seqlens_kv[b]) // wl.block_size)]] = True
    free = np.flatnonzero(~used)
    for x in free[:: max(1, len(free) // 8)][:8]:
        assert (_bits(d["kc"][int(x)]) == NAN_BITS).all()


def _new_token_values(wl, vals):
    rows = torch.from_numpy(wl.new_rows).to(vals["k_all"].device)
    return vals["k_all"][rows].contiguous(), vals["v_all"][rows].contiguous()


@pytest.mark.parametrize("make", [W.tiny, lambda: W.small((16, 4), (64, 32), 8, 2),
                                  lambda: W.custom([3, 0, 1, 7], [40, 5, 1, 300], 8, 2, 128, 16,
                                                   dtype="bf16")])
def test_scatter_paged_bit_exact_small(make):
    """Slots derived on the GPU from (cu_seqlens_q, seqlens_kv, block_table)
    write exactly the bytes the oracle's in-op addressing says, into
    NaN-filled caches; a negative table entry skips its tokens."""
    wl = make()
    _log(f"scatter paged: {wl.name}")
    require_gpu()
    vals = {k: v.cuda() for k, v in W.make_values(wl).items()}
    k_new, v_new = _new_token_values(wl, vals)
    table = wl.block_table.astype(np.int32).copy()
    # Drop the block of the first new token of the last non-empty sequence.
    b_last = int(np.flatnonzero(wl.q_lens > 0)[-1])
    pos0 = int(wl.seqlens_kv[b_last] - wl.q_lens[b_last])
    table[b_last, pos0 // wl.block_size] = -1
    slots = oracle.slots_from_block_table(wl.cu_seqlens_q, wl.seqlens_kv, table, wl.block_size)
    shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_size)
    kref = np.full(shape, NAN_BITS, dtype=np.uint16)
    vref = np.full(shape, NAN_BITS, dtype=np.uint16)
    slots[slots < 0] = -1    # tokens whose table entry is negative are skipped
    oracle.scatter_kv(_bits(k_new), _bits(v_new), slots, kref, vref, wl.block_size)
    kc, vc = nan_cache(wl), nan_cache(wl)
    pa.pa_scatter_kv_paged(k_new, v_new, torch.from_numpy(wl.cu_seqlens_q).cuda(),
                           torch.from_numpy(wl.seqlens_kv.astype(np.int32)).cuda(),
                           torch.from_numpy(table).cuda(), kc, vc)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(kc), kref)
    assert np.array_equal(_bits(vc), vref)


@pytest.mark.parametrize("idx", [3, 5])
def test_scatter_paged_large(idx):
    """Multi-GB pools: the device-derived slots land where the slot-mapping
    scatter puts the same tokens (sign-flipped values over the filled
    cache), bit for bit on sampled sequences' blocks."""
    wl = W.by_index(idx)
    _log(f"scatter paged: {wl.name}")
    d = device_inputs(wl, backend="torch")
    k_new, v_new = _new_token_values(wl, d)
    k_neg = (k_new.view(torch.int16) ^ -0x8000).view(k_new.dtype)   # sign bit flipped
    v_neg = (v_new.view(torch.int16) ^ -0x8000).view(v_new.dtype)
    pa.pa_scatter_kv_paged(k_neg, v_neg, d["cu"], d["lens"], d["table"], d["kc"], d["vc"])
    torch.cuda.synchronize()
    slots = oracle.slots_from_block_table(wl.cu_seqlens_q, wl.seqlens_kv, wl.block_table,
                                          wl.block_size)
    assert np.array_equal(slots, wl.slot_mapping.astype(np.int64))
    rng = np.random.default_rng(100 + idx)
    seqs = [int(x) for x in rng.choice(np.flatnonzero(wl.q_lens > 0), size=4, replace=False)]
    kv_cu, cu = wl.kv_cu, wl.cu_seqlens_q
    shape = (wl.block_size, wl.num_kv_heads, wl.head_size)
    kb_new, vb_new = _bits(k_neg), _bits(v_neg)
    for b in seqs:
        nb = -(-int(wl.seqlens_kv[b]) // wl.block_size)
        blocks = [int(x) for x in wl.block_table[b, :nb]]
        kref = {x: np.full(shape, NAN_BITS, dtype=np.uint16) for x in blocks}
        vref = {x: np.full(shape, NAN_BITS, dtype=np.uint16) for x in blocks}
        oracle.scatter_kv(_bits(d["k_all"][kv_cu[b]:kv_cu[b + 1]]),
                          _bits(d["v_all"][kv_cu[b]:kv_cu[b + 1]]),
                          wl.kv_slots[kv_cu[b]:kv_cu[b + 1]], kref, vref, wl.block_size)
        oracle.scatter_kv(kb_new[cu[b]:cu[b + 1]], vb_new[cu[b]:cu[b + 1]], slots[cu[b]:cu[b + 1]],
                          kref, vref, wl.block_size)
        for x in blocks:
            assert np.array_equal(_bits(d["kc"][x]), kref[x]), (b, x)
            assert np.array_equal(_bits(d["vc"][x]), vref[x]), (b, x)


def test_seqlens_from_past():
    require_gpu()
    rng = np.random.default_rng(7)
    q_lens = rng.integers(0, 40, size=3000).astype(np.int32)
    past = rng.integers(0, 100000, size=3000).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    out = pa.pa_seqlens_from_past(torch.from_numpy(cu).cuda(), torch.from_numpy(past).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), past + q_lens)


# ---------------------------------------------------------------- attention

def test_tiny_mixed_batch():
    wl = W.tiny()
    _log(f"attention: {wl.name}")
    d = device_inputs(wl)
    out = run_attention(wl, d)
    ref = oracle_full(wl, d)
    assert np.isfinite(to_np64(out)).all()
    assert max_err(out, ref) <= TOL[wl.dtype]


def test_small_matrix_all_cases():
    """The 84-case small matrix (MHA and GQA, q_len {1,4,16}, total {32,64},
    block 256, batch 1 and 2)."""
    worst = 0.0
    for n, (qs, ls, hq, hk) in enumerate(W.small_cases()):
        wl = W.small(qs, ls, hq, hk, seed=2000 + n)
        d = device_inputs(wl)
        out = run_attention(wl, d)
        err = max_err(out, oracle_full(wl, d))
        worst = max(worst, err)
        assert err <= TOL[wl.dtype], (n, wl.name, err)
    _log(f"small matrix worst error {worst:.3g}")


@pytest.mark.parametrize("idx", [3, 4, 5])
def test_large_workloads_sampled(idx):
    """Full-size workloads in the benchmarked launch configuration; outputs
    checked on sampled rows (first, last and random rows of sampled
    sequences) against the oracle, all outputs finite."""
    wl = W.by_index(idx)
    _log(f"attention: {wl.name}")
    d = device_inputs(wl, backend="torch")
    out = run_attention(wl, d)
    assert torch.isfinite(out).all()
    rng = np.random.default_rng(100 + idx)
    picks = []
    pre = np.flatnonzero(wl.q_lens > 1)
    dec = np.flatnonzero(wl.q_lens == 1)
    for b in rng.choice(dec, size=min(6, len(dec)), replace=False) if len(dec) else []:
        picks.append((int(b), 0))
    longest = int(np.argmax(np.where(wl.q_lens == 1, wl.seqlens_kv, -1))) if len(dec) else None
    if longest is not None:
        picks.append((longest, 0))
    for b in rng.choice(pre, size=min(2, len(pre)), replace=False) if len(pre) else []:
        ql = int(wl.q_lens[b])
        rows = {0, 1, ql - 1} | set(int(x) for x in rng.choice(ql, size=5, replace=False))
        picks += [(int(b), i) for i in sorted(rows)]
    ref, toks = oracle_rows(wl, d, picks)
    err = max_err(out[torch.from_numpy(toks).cuda()], ref)
    _log(f"  {len(picks)} sampled rows, max error {err:.3g}")
    assert err <= TOL[wl.dtype]


@pytest.mark.parametrize("name", ["flex_attention_basic.txt", "flex_attention_gqa.txt"])
def test_printed_examples_on_gpu(name):
    """The FlexAttention page's examples through the paged path (D padded to
    64 with zeros): within fp16 tolerance of the printed Y."""
    require_gpu()
    e = embed_flex_example(load_golden(name), pad_to=64)
    dt = torch.float16
    q = torch.from_numpy(e["q"]).to(dt).cuda()
    kc = torch.from_numpy(e["k_cache"]).to(dt).cuda()
    vc = torch.from_numpy(e["v_cache"]).to(dt).cuda()
    out = pa.pa_attention(q, torch.from_numpy(e["cu"]).cuda(),
                          torch.from_numpy(e["seqlens_kv"]).cuda(),
                          torch.from_numpy(e["block_table"]).cuda(), kc, vc, e["scale"],
                          e["num_heads"], e["num_kv_heads"])
    torch.cuda.synchronize()
    assert np.abs(to_np64(out) - e["y"]).max() <= 2e-3


def test_first_token_returns_value_row_exactly():
    """q_len 1, past 0: the output is V row 0 of the KV head, bit for bit."""
    wl = W.custom([1, 1], [1, 1], 8, 2, 128, 16, seed=3)
    d = device_inputs(wl)
    out = run_attention(wl, d)
    G = wl.num_heads // wl.num_kv_heads
    for b in range(2):
        v = d["v_all"][wl.kv_cu[b]]
        for h in range(wl.num_heads):
            assert torch.equal(out[b, h], v[h // G])


@pytest.mark.parametrize("q_lens,lens", [([1, 3, 1], [700, 40, 1300]), ([37, 1], [2000, 600])])
def test_gqa_mapping_constant_values(q_lens, lens):
    """V of KV head k filled with the constant k: every output of query head
    h is exactly floor(h / G), on the decode and prefill paths."""
    wl = W.custom(q_lens, lens, 16, 4, 128, 16, seed=4)
    d = device_inputs(wl)
    for k in range(wl.num_kv_heads):
        d["v_all"][:, k, :] = float(k)
    pa.pa_scatter_kv(d["k_all"], d["v_all"], d["slots_all"], d["kc"], d["vc"])
    out = run_attention(wl, d)
    G = wl.num_heads // wl.num_kv_heads
    for h in range(wl.num_heads):
        assert (out[:, h].float() == float(h // G)).all()


@pytest.mark.parametrize("q_lens,lens,hq,hk", [([4, 1], [900, 1030], 16, 4),     # decode path
                                               ([300], [700], 8, 2)])            # prefill path
def test_causality_bitwise(q_lens, lens, hq, hk):
    """Changing K/V at positions beyond past + i leaves row i bit-identical;
    changing a visible position changes it."""
    wl = W.custom(q_lens, lens, hq, hk, 128, 16, seed=5)
    d = device_inputs(wl)
    base = run_attention(wl, d).clone()
    b = 0
    past = int(lens[b] - q_lens[b])
    cut = past + q_lens[b] // 2            # rows i <= cut - past keep their output
    kv0 = int(wl.kv_cu[b])
    k2, v2 = d["k_all"].clone(), d["v_all"].clone()
    k2[kv0 + cut + 1: kv0 + lens[b]] *= -1.5
    v2[kv0 + cut + 1: kv0 + lens[b]] += 0.75
    pa.pa_scatter_kv(k2, v2, d["slots_all"], d["kc"], d["vc"])
    out = run_attention(wl, d)
    keep = cut - past + 1
    assert torch.equal(out[:keep], base[:keep])
    if keep < q_lens[b]:
        assert not torch.equal(out[keep:q_lens[b]], base[keep:q_lens[b]])
    assert torch.equal(out[q_lens[b]:], base[q_lens[b]:])   # other sequences untouched


def test_block_placement_invariance_bitwise():
    """Same sequences, different physical blocks: bit-identical outputs
    (a sequence's result never depends on where its blocks live)."""
    wl1 = W.custom([1, 20, 1], [3000, 500, 17], 32, 8, 128, 16, seed=6)
    wl2 = W.custom([1, 20, 1], [3000, 500, 17], 32, 8, 128, 16, seed=6)
    perm = np.random.default_rng(1).permutation(wl1.num_blocks)
    wl2.block_table = np.where(wl1.block_table >= 0, perm[wl1.block_table], -1).astype(np.int32)
    d1, d2 = device_inputs(wl1), device_inputs(wl2)
    assert torch.equal(d1["q"], d2["q"])
    assert torch.equal(run_attention(wl1, d1), run_attention(wl2, d2))


def test_batch_invariance_bitwise():
    """A sequence's output does not depend on its batch-mates."""
    wl = W.custom([1, 9, 1], [2100, 60, 40], 32, 8, 128, 16, seed=8)
    d = device_inputs(wl)
    full = run_attention(wl, d)
    one = W.custom([1], [2100], 32, 8, 128, 16, seed=8)
    one.block_table = wl.block_table[:1].copy()
    one.num_blocks = wl.num_blocks
    d1 = dict(d)
    d1["q"] = d["q"][:1]
    d1["cu"] = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    d1["lens"] = d["lens"][:1].contiguous()
    d1["table"] = d["table"][:1].contiguous()
    out1 = pa.pa_attention(d1["q"], d1["cu"], d1["lens"], d1["table"], d["kc"], d["vc"], wl.scale,
                           wl.num_heads, wl.num_kv_heads)
    torch.cuda.synchronize()
    assert torch.equal(out1[0], full[0])


# ---------------------------------------------------------------- edge cases

EDGE = [
    # (q_lens, total kv, Hq, Hk, D, block size, dtype)
    ([1], [1], 4, 4, 64, 16, "f16"),
    ([0, 3, 0, 1], [5, 3, 0, 9], 8, 2, 64, 16, "f16"),            # empty sequences
    ([1, 1, 1, 1, 1], [512, 513, 1024, 1025, 2048], 32, 8, 128, 16, "f16"),   # split boundaries
    ([1, 1], [1, 4097], 64, 8, 128, 16, "bf16"),
    ([4, 2, 16], [1500, 2, 16], 16, 4, 128, 32, "f16"),           # q_len*G = 16 decode path
    ([5, 17], [1600, 17], 16, 4, 128, 64, "bf16"),                # q_len*G > 16 prefill path
    ([16, 16], [16, 1100], 16, 16, 128, 16, "f16"),               # MHA, 16 columns
    ([130, 1], [130, 77], 8, 8, 64, 256, "f16"),                  # MHA prefill, D 64
    ([33], [100], 12, 4, 128, 16, "f16"),                         # G = 3 (tile rows padded)
    ([9, 1], [9, 3000], 128, 1, 128, 16, "bf16"),                 # G = 128
    ([200, 1, 70], [1200, 9000, 70], 32, 8, 128, 1024, "f16"),    # block 1024
    ([64, 1], [64, 700], 8, 1, 64, 128, "bf16"),
]


@pytest.mark.parametrize("case", EDGE, ids=[str(i) for i in range(len(EDGE))])
def test_edge_cases(case):
    q_lens, lens, hq, hk, dd, bs, dt = case
    wl = W.custom(q_lens, lens, hq, hk, dd, bs, dtype=dt, seed=11)
    _log(f"edge: {wl.name}")
    d = device_inputs(wl)
    out = run_attention(wl, d)
    ref = oracle_full(wl, d)
    assert np.isfinite(to_np64(out)).all()
    assert max_err(out, ref) <= TOL[dt]


def test_empty_call_and_repeat_determinism():
    wl = W.custom([3, 1], [50, 2000], 32, 8, 128, 16, seed=12)
    d = device_inputs(wl)
    a1 = run_attention(wl, d).clone()
    a2 = run_attention(wl, d)
    assert torch.equal(a1, a2)
    empty = torch.empty((0, wl.num_heads, wl.head_size), dtype=torch.float16, device="cuda")
    out = pa.pa_attention(empty, torch.zeros(2, dtype=torch.int32, device="cuda"), d["lens"][:1],
                          d["table"][:1], d["kc"], d["vc"], wl.scale, wl.num_heads,
                          wl.num_kv_heads)
    assert out.shape[0] == 0


def test_validate_metadata_through_abi():
    wl = W.tiny()
    d = device_inputs(wl)
    assert pa.pa_validate_metadata(d["cu"], d["lens"], d["table"], wl.num_blocks, wl.block_size,
                                   slot_mapping=d["slots_new"], num_tokens=wl.num_tokens) == 0
    bad = d["table"].clone()
    bad[0, 0] = wl.num_blocks
    assert pa.pa_validate_metadata(d["cu"], d["lens"], bad, wl.num_blocks,
                                   wl.block_size) & (1 << 5)
    dup = d["slots_new"].clone()
    dup[1] = dup[2]
    assert pa.pa_validate_metadata(d["cu"], d["lens"], d["table"], wl.num_blocks, wl.block_size,
                                   slot_mapping=dup, num_tokens=wl.num_tokens) & (1 << 7)


def test_longest_context():
    """The longest context the decode path takes (262144 keys = 256 splits,
    all combined) with 16 columns (q_len 2, G 8), beside a prefill-path
    chunk over 32768 keys; plain and with a cap and a window."""
    wl = W.custom([2, 24], [262144, 32768], 8, 1, 128, 256, dtype="bf16", seed=13)
    _log(f"longest context: {wl.name}")
    d = device_inputs(wl, backend="torch")
    q = to_np64(d["q"])
    kc, vc = oracle_caches(wl, to_np64(d["k_all"]), to_np64(d["v_all"]))
    for opts in ({}, {"softcap": 30.0, "local_window_size": 70000}):
        out = run_attention(wl, d, **opts)
        ref = oracle.attention(q, wl.cu_seqlens_q, wl.seqlens_kv, wl.block_table, kc, vc,
                               wl.scale, wl.num_heads, wl.num_kv_heads, wl.block_size, **opts)
        assert np.isfinite(to_np64(out)).all()
        assert max_err(out, ref) <= TOL["bf16"], opts


def test_maximum_sequence_count():
    """65536 sequences (the largest batch the boundary accepts): empty
    sequences, decodes, 2- and 3-token rows and 20-token prefill chunks over
    short contexts, checked on sampled rows including the batch's last."""
    rng = np.random.default_rng(21)
    B = 65536
    q_lens = rng.choice([0, 1, 1, 1, 2, 3, 20], size=B).astype(np.int32)
    lens = q_lens + rng.integers(0, 40, size=B, endpoint=True)
    lens[q_lens == 0] = 0
    q_lens[-1], lens[-1] = 3, 45
    wl = W.custom(q_lens, lens, 8, 2, 64, 16, dtype="f16", seed=21)
    _log(f"maximum sequence count: {B} sequences, {wl.num_tokens} tokens")
    d = device_inputs(wl, backend="torch")
    out = run_attention(wl, d)
    live = np.flatnonzero(wl.q_lens > 0)
    picks = [(int(b), int(rng.integers(0, wl.q_lens[b]))) for b in rng.choice(live, 200, replace=False)]
    picks += [(int(live[0]), 0), (B - 1, 0), (B - 1, 2)]
    ref, toks = oracle_rows(wl, d, picks)
    assert np.isfinite(to_np64(out)).all()
    assert max_err(out[torch.from_numpy(toks).cuda()], ref) <= TOL["f16"]


def test_plan_past_one_sweep():
    """1100 sequences, more than one sweep of the plan's 1024-thread
    work-group, so the plan places the partial last decode splits and the
    prefill items in a second sweep: decodes over contexts of up to four
    1024-key splits (most with a partial last split), 20-token prefill
    chunks and empty sequences.  Every row against the oracle; and each half
    of the batch (550 sequences, planned in one sweep) run alone over the
    same cache gives bitwise its rows of the whole batch."""
    rng = np.random.default_rng(23)
    B = 1100
    kind = rng.choice([0, 1, 1, 1, 2], size=B)            # empty, decode x3, prefill chunk
    q_lens = np.where(kind == 0, 0, np.where(kind == 1, 1, 20)).astype(np.int32)
    lens = np.where(kind == 1, rng.integers(1, 4096, size=B, endpoint=True),
                    np.where(kind == 2, 20 + rng.integers(0, 300, size=B), 0)).astype(np.int64)
    wl = W.custom(q_lens, lens, 8, 2, 64, 16, dtype="f16", seed=23)
    _log(f"plan past one sweep: {B} sequences, {wl.num_tokens} tokens, "
         f"{int(((lens + 1023) // 1024 > 1).sum())} multi-split decodes")
    d = device_inputs(wl, backend="torch")
    out = run_attention(wl, d)
    assert max_err(out, oracle_full(wl, d)) <= TOL["f16"]
    cu = wl.cu_seqlens_q
    for b0, b1 in ((0, B // 2), (B // 2, B)):
        sub_cu = torch.from_numpy((cu[b0:b1 + 1] - cu[b0]).astype(np.int32)).cuda()
        q = d["q"][int(cu[b0]):int(cu[b1])].contiguous()
        part = pa.pa_attention(q, sub_cu, d["lens"][b0:b1].contiguous(),
                               d["table"][b0:b1].contiguous(), d["kc"], d["vc"], wl.scale,
                               wl.num_heads, wl.num_kv_heads)
        torch.cuda.synchronize()
        assert torch.equal(part, out[int(cu[b0]):int(cu[b1])]), (b0, b1)


def test_concurrent_calls_on_two_streams():
    """Two batches on two streams with their own workspaces, launches
    interleaved: each output is bitwise the one its batch gets alone."""
    wl1 = W.custom([1, 40, 1, 3], [3000, 500, 20, 2100], 32, 8, 128, 16, seed=31)
    wl2 = W.custom([2, 1, 17, 1], [5000, 70, 900, 1025], 32, 8, 128, 16, dtype="bf16", seed=32)
    _log(f"two streams: {wl1.name} | {wl2.name}")
    runs = []
    for wl in (wl1, wl2):
        d = device_inputs(wl)
        ref = run_attention(wl, d).clone()
        need = pa.pa_attention_workspace_size(wl.num_seqs, wl.num_tokens, wl.max_blocks_per_seq,
                                              wl.num_heads, wl.num_kv_heads, wl.head_size,
                                              wl.block_size)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        runs.append((wl, d, ref, torch.empty_like(ref), ws, torch.cuda.Stream()))
    torch.cuda.synchronize()
    for _ in range(4):
        for wl, d, _, out, ws, st in runs:
            pa.pa_attention(d["q"], d["cu"], d["lens"], d["table"], d["kc"], d["vc"], wl.scale,
                            wl.num_heads, wl.num_kv_heads, out=out, workspace=ws, stream=st)
    torch.cuda.synchronize()
    for wl, _, ref, out, _, _ in runs:
        assert torch.equal(out, ref), wl.name


def test_default_workspace_on_side_streams():
    """Calls on side streams that leave out and workspace to the binding:
    the binding allocates both on the call's stream, so allocations made on
    the current stream right after each call (filled with zeros, which keep
    every work-list index in range) never take the bytes of a workspace that
    a side-stream kernel still uses.  Every output is bitwise its batch's
    solo output."""
    wl1 = W.custom([1, 40, 1, 3], [3000, 500, 20, 2100], 32, 8, 128, 16, seed=33)
    wl2 = W.custom([2, 1, 17, 1], [5000, 70, 900, 1025], 32, 8, 128, 16, dtype="bf16", seed=34)
    _log(f"default workspace on side streams: {wl1.name} | {wl2.name}")
    runs = []
    for wl in (wl1, wl2):
        d = device_inputs(wl)
        runs.append((wl, d, run_attention(wl, d).clone(), torch.cuda.Stream()))
    torch.cuda.synchronize()
    outs, junk = [], []
    for _ in range(4):
        for wl, d, _, st in runs:
            st.wait_stream(torch.cuda.current_stream())
            o = pa.pa_attention(d["q"], d["cu"], d["lens"], d["table"], d["kc"], d["vc"],
                                wl.scale, wl.num_heads, wl.num_kv_heads, stream=st)
            outs.append((wl.name, o))
            junk.append(torch.zeros(1 << 22, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    refs = {wl.name: ref for wl, _, ref, _ in runs}
    for name, o in outs:
        assert torch.equal(o, refs[name]), name


def test_step_under_graph_capture():
    """The scatter of new rows plus the attention, captured in one graph
    (caller-owned output and workspace; the entry points only launch
    kernels): each replay, with eager work and synchronisation between
    replays, equals the eager step bitwise."""
    wl = W.custom([1, 40, 1, 3], [3000, 500, 20, 2100], 32, 8, 128, 16, seed=41)
    _log(f"graph capture: {wl.name}")
    d = device_inputs(wl)
    rows = torch.from_numpy(wl.new_rows).cuda()
    k_new, v_new = d["k_all"][rows].contiguous(), d["v_all"][rows].contiguous()
    need = pa.pa_attention_workspace_size(wl.num_seqs, wl.num_tokens, wl.max_blocks_per_seq,
                                          wl.num_heads, wl.num_kv_heads, wl.head_size,
                                          wl.block_size)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["q"])

    def step():
        pa.pa_scatter_kv(k_new, v_new, d["slots_new"], d["kc"], d["vc"])
        pa.pa_attention(d["q"], d["cu"], d["lens"], d["table"], d["kc"], d["vc"], wl.scale,
                        wl.num_heads, wl.num_kv_heads, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
