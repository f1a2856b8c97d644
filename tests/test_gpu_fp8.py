"""Parity of the fp8 (e4m3) KV-cache path (pa_scatter_kv_fp8,
pa_attention_fp8, through the C ABI) with the fp8 oracle (oracle/kv_fp8.py).

Bars: every cache byte bit-exact (the quantization is fixed by its
definition, both sides round in float32); attention within the 16-bit
path's bars (max abs 2e-3 fp16, 1.6e-2 bf16) of the oracle over the
dequantized cache.  Unused cache slots hold NaN codes, so any read of them
shows up as a non-finite output.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_pa_amd import workloads as W
from gpu_util import (FP8_NAN, TOL, device_inputs_fp8, max_err, oracle_codes_fp8,
                      oracle_codes_fp8_for, oracle_full_fp8, oracle_rows_fp8, run_attention_fp8)

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


SMALL = [
    ("tiny", W.tiny),
    ("decode f16 D128 bs16, 1-3 splits", lambda: W.custom([1, 1, 1, 1], [5, 1024, 1025, 2600],
                                                          16, 4, 128, 16)),
    ("speculative 4 x G4 bf16 D128 bs32", lambda: W.custom([4, 2, 1, 4], [4, 700, 2049, 3000], 16,
                                                           4, 128, 32, dtype="bf16")),
    ("MHA q_len 16 f16 D64 bs16", lambda: W.custom([16, 3, 1], [16, 900, 1500], 4, 4, 64, 16)),
    ("G16 f16 D128 bs64", lambda: W.custom([1, 1, 1], [33, 1100, 4097], 32, 2, 128, 64)),
    ("G8 bf16 D64 bs16, empty sequence", lambda: W.custom([2, 0, 1, 2], [300, 17, 1, 2000], 16, 2,
                                                          64, 16, dtype="bf16")),
]


@pytest.mark.parametrize("name,make", SMALL, ids=[s[0] for s in SMALL])
def test_scatter_fp8_bit_exact_small(name, make):
    wl = make()
    _log(f"fp8 scatter: {wl.name}")
    d = device_inputs_fp8(wl)
    kc, vc = oracle_codes_fp8(wl, d)
    np.testing.assert_array_equal(d["kc"].cpu().numpy(), kc)
    np.testing.assert_array_equal(d["vc"].cpu().numpy(), vc)


def test_scatter_fp8_large_sampled():
    """The pure-decode pool (2 x 2.1 GB of codes): sampled sequences' blocks
    bit-exact, and blocks no sequence uses still hold NaN codes."""
    wl = W.by_index(3)
    _log(f"fp8 scatter: {wl.name}")
    d = device_inputs_fp8(wl, backend="torch")
    rng = np.random.default_rng(31)
    seqs = [int(b) for b in rng.choice(wl.num_seqs, size=6, replace=False)]
    kc, vc = oracle_codes_fp8_for(wl, d, seqs)
    for blk in kc:
        np.testing.assert_array_equal(d["kc"][blk].cpu().numpy(), kc[blk])
        np.testing.assert_array_equal(d["vc"][blk].cpu().numpy(), vc[blk])
    used = np.zeros(wl.num_blocks, bool)
    for b in range(wl.num_seqs):
        used[wl.block_table[b, :-(-int(wl.seqlens_kv[b]) // wl.block_size)]] = True
    free = np.flatnonzero(~used)
    assert len(free) > 0
    assert (d["kc"][torch.from_numpy(free[:3]).cuda()] == FP8_NAN).all()


@pytest.mark.parametrize("name,make", SMALL, ids=[s[0] for s in SMALL])
def test_attention_fp8_small(name, make):
    wl = make()
    _log(f"fp8 attention: {wl.name}")
    d = device_inputs_fp8(wl)
    out = run_attention_fp8(wl, d)
    assert torch.isfinite(out).all()
    err = max_err(out, oracle_full_fp8(wl, d))
    _log(f"  max error {err:.3g}")
    assert err <= TOL[wl.dtype]


def test_attention_fp8_decode_workload_sampled():
    """The full pure-decode workload on fp8 caches, in the benchmarked launch
    configuration; sampled rows (random and the longest sequences) against
    the oracle."""
    wl = W.by_index(3)
    _log(f"fp8 attention: {wl.name}")
    d = device_inputs_fp8(wl, backend="torch")
    out = run_attention_fp8(wl, d)
    assert torch.isfinite(out).all()
    rng = np.random.default_rng(32)
    picks = [(int(b), 0) for b in rng.choice(wl.num_seqs, size=8, replace=False)]
    picks.append((int(np.argmax(wl.seqlens_kv)), 0))
    ref, toks = oracle_rows_fp8(wl, d, picks)
    err = max_err(out[torch.from_numpy(toks).cuda()], ref)
    _log(f"  {len(picks)} sampled rows, max error {err:.3g}")
    assert err <= TOL[wl.dtype]


def test_attention_fp8_repeat_is_bitwise_identical():
    wl = SMALL[1][1]()
    d = device_inputs_fp8(wl)
    a = run_attention_fp8(wl, d)
    b = run_attention_fp8(wl, d)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_attention_fp8_precondition_violation_leaves_rows():
    """A sequence whose q_len * G exceeds 16 although max_q_len claims
    otherwise gets no work: its rows keep what the output held; the other
    sequences are still right."""
    wl = W.custom([1, 5, 1], [40, 60, 1030], 16, 4, 128, 16)   # q_len 5 * G 4 = 20 > 16
    d = device_inputs_fp8(wl)
    out = torch.full((wl.num_tokens, wl.num_heads, wl.head_size), 7.0, dtype=torch.float16,
                     device="cuda")
    run_attention_fp8(wl, d, max_q_len=1, out=out)
    cu = wl.cu_seqlens_q
    assert (out[cu[1]:cu[2]] == 7.0).all()
    ref = oracle_full_fp8(wl, d)
    keep = np.r_[cu[0]:cu[1], cu[2]:cu[3]]
    err = max_err(out[torch.from_numpy(keep).cuda()], ref[keep])
    assert err <= TOL[wl.dtype]


def test_attention_fp8_longest_context():
    """fp8 caches at the longest decode context (262144 keys, 256 splits)
    with 16 columns (q_len 2, G 8) and a 1-token decode beside it; plain and
    with a cap and a window."""
    wl = W.custom([2, 1], [262144, 200000], 8, 1, 128, 256, dtype="bf16", seed=17)
    _log(f"fp8 longest context: {wl.name}")
    d = device_inputs_fp8(wl, backend="torch")
    for opts in ({}, {"softcap": 30.0, "local_window_size": 70000}):
        out = run_attention_fp8(wl, d, **opts)
        assert torch.isfinite(out).all()
        err = max_err(out, oracle_full_fp8(wl, d, **opts))
        _log(f"  {opts} max error {err:.3g}")
        assert err <= TOL["bf16"], opts
