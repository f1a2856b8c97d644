"""Parity of the sliding window (local_window_size) and the score soft cap
(softcap) through the C ABI with the oracle's options of the same names.

Bars as for plain attention: max abs error 2e-3 (fp16) / 1.6e-2 (bf16)
against the fp64 oracle.  The caps used here (0.7 .. 5) bend the scaled
scores of these inputs (|x| up to ~3) well away from the identity, so a
missing or misplaced cap fails; the windows land on, beside and across the
64-key tile and 1024-key split boundaries.  Unused cache slots hold NaN;
one test also puts NaN into the keys and values that the kernels skip
(whole splits and tiles before a sequence's first window), so reading them
would show up as a non-finite output.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_pa_amd as pa
from paged_kv_cache_pa_amd import workloads as W
from gpu_util import (TOL, device_inputs, device_inputs_fp8, max_err, oracle_full,
                      oracle_full_fp8, oracle_rows, oracle_rows_fp8, run_attention,
                      run_attention_fp8)

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _prefill_g4():
    # G 4: 64 tokens per prefill tile; sequences with ragged tails, one with
    # no history, one decode row.
    return W.custom([300, 77, 1, 130], [300, 2100, 3000, 130], 16, 4, 128, 16)


def _decode_splits():
    # decode rows over 1 .. 5 splits of 1024 keys
    return W.custom([1, 1, 1, 1, 1], [5, 1100, 2600, 4097, 5000], 16, 4, 128, 16)


CASES = [
    ("tiny W1", W.tiny, 0.0, 1),
    ("tiny W5 cap0.7", W.tiny, 0.7, 5),
    ("tiny cap5", W.tiny, 5.0, 0),
    ("prefill G4 W1", _prefill_g4, 0.0, 1),
    ("prefill G4 W63", _prefill_g4, 0.0, 63),
    ("prefill G4 W64", _prefill_g4, 0.0, 64),
    ("prefill G4 W65", _prefill_g4, 0.0, 65),
    ("prefill G4 W257 cap1", _prefill_g4, 1.0, 257),
    ("prefill G4 W2000", _prefill_g4, 0.0, 2000),
    ("prefill G4 cap0.7", _prefill_g4, 0.7, 0),
    ("decode W1", _decode_splits, 0.0, 1),
    ("decode W100", _decode_splits, 0.0, 100),
    ("decode W1024 cap2", _decode_splits, 2.0, 1024),
    ("decode W1500", _decode_splits, 0.0, 1500),
    ("decode W3000 cap0.7", _decode_splits, 0.7, 3000),
    ("speculative 4 x G4 bf16 W300 cap1.5",
     lambda: W.custom([4, 2, 1, 4], [4, 700, 2049, 3000], 16, 4, 128, 32, dtype="bf16"), 1.5, 300),
    ("MHA bf16 D64 bs32 W150 cap2",
     lambda: W.custom([200, 1, 33], [900, 700, 33], 4, 4, 64, 32, dtype="bf16"), 2.0, 150),
    ("G8 bf16 D64 W500",
     lambda: W.custom([40, 2, 1], [1500, 2000, 17], 16, 2, 64, 16, dtype="bf16"), 0.0, 500),
    ("G16 D128 bs64 W700 cap5",
     lambda: W.custom([1, 1, 16, 20], [33, 4097, 3000, 1200], 32, 2, 128, 64), 5.0, 700),
]


@pytest.mark.parametrize("name,make,cap,win", CASES, ids=[c[0] for c in CASES])
def test_window_softcap_small(name, make, cap, win):
    wl = make()
    _log(f"attention softcap={cap} window={win}: {wl.name}")
    d = device_inputs(wl)
    out = run_attention(wl, d, softcap=cap, local_window_size=win)
    assert torch.isfinite(out).all()
    err = max_err(out, oracle_full(wl, d, softcap=cap, local_window_size=win))
    _log(f"  max error {err:.3g}")
    assert err <= TOL[wl.dtype]


# The plain-attention edge cases (empty sequences, split boundaries, the
# q_len * G = 16 / 17 path switch, MHA, G = 3, G = 128, block 1024, D 64)
# with a short window and a cap, and with a longer window alone.
from test_gpu_parity import EDGE  # noqa: E402

EDGE_OPTS = [(1.5, 37), (0.0, 300)]


@pytest.mark.parametrize("case", EDGE, ids=[str(i) for i in range(len(EDGE))])
@pytest.mark.parametrize("cap,win", EDGE_OPTS, ids=["cap1.5-W37", "W300"])
def test_window_softcap_edge_cases(case, cap, win):
    q_lens, lens, hq, hk, dd, bs, dt = case
    wl = W.custom(q_lens, lens, hq, hk, dd, bs, dtype=dt, seed=11)
    _log(f"edge softcap={cap} window={win}: {wl.name}")
    d = device_inputs(wl)
    out = run_attention(wl, d, softcap=cap, local_window_size=win)
    assert torch.isfinite(out).all()
    assert max_err(out, oracle_full(wl, d, softcap=cap, local_window_size=win)) <= TOL[dt]


def test_options_change_the_result():
    """The options are not silently ignored: each moves the output far
    beyond the tolerance on the same inputs."""
    wl = _prefill_g4()
    d = device_inputs(wl)
    base = run_attention(wl, d).float()
    for kw in (dict(softcap=0.7), dict(local_window_size=63)):
        assert (run_attention(wl, d, **kw).float() - base).abs().max().item() > 0.05


@pytest.mark.parametrize("make,win", [(_prefill_g4, 65), (_decode_splits, 100),
                                      (lambda: W.custom([1, 1, 16, 20], [33, 4097, 3000, 1200],
                                                        32, 2, 128, 64), 700)])
def test_skipped_units_are_not_read(make, win):
    """K/V slots before the window are skipped in whole units: 1024-key
    splits for decode-path rows (q_len * G <= 16), 64-key tiles for prefill
    rows (the unit holding the first row's first visible key and later
    ones are read).  NaN written into the skipped slots leaves the output
    finite and unchanged."""
    wl = make()
    d = device_inputs(wl)
    want = run_attention(wl, d, local_window_size=win)
    slots = []
    for b in range(wl.num_seqs):
        ql, L = int(wl.q_lens[b]), int(wl.seqlens_kv[b])
        unit = 1024 if ql * wl.num_heads // wl.num_kv_heads <= 16 else 64
        skip = max(0, L - ql - win + 1) // unit * unit
        slots += list(wl.kv_slots[wl.kv_cu[b]:wl.kv_cu[b] + skip])
    assert len(slots) > 0
    nan = torch.full((len(slots), wl.num_kv_heads, wl.head_size), float("nan"),
                     dtype=d["kc"].dtype, device="cuda")
    pa.pa_scatter_kv(nan, nan, torch.tensor(slots, dtype=torch.int32, device="cuda"), d["kc"],
                     d["vc"])
    got = run_attention(wl, d, local_window_size=win)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_window_covering_everything_is_bitwise_plain():
    """A window at least as long as every context takes the same path as no
    window: bitwise identical outputs on the full large mixed batch."""
    wl = W.by_index(5)
    _log(f"attention window >= every length: {wl.name}")
    d = device_inputs(wl, backend="torch")
    a = run_attention(wl, d)
    b = run_attention(wl, d, local_window_size=int(wl.seqlens_kv.max()))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _picks(wl, rng):
    picks = []
    pre = np.flatnonzero(wl.q_lens > 1)
    dec = np.flatnonzero(wl.q_lens == 1)
    if len(dec):
        picks += [(int(b), 0) for b in rng.choice(dec, size=min(6, len(dec)), replace=False)]
        picks.append((int(np.argmax(np.where(wl.q_lens == 1, wl.seqlens_kv, -1))), 0))
    for b in rng.choice(pre, size=min(2, len(pre)), replace=False) if len(pre) else []:
        ql = int(wl.q_lens[b])
        rows = {0, 1, ql - 1} | set(int(x) for x in rng.choice(ql, size=5, replace=False))
        picks += [(int(b), i) for i in sorted(rows)]
    return picks


@pytest.mark.parametrize("idx,cap,win", [(5, 0.8, 777), (4, 0.0, 1024), (3, 1.0, 2000)])
def test_window_softcap_large_sampled(idx, cap, win):
    """Full-size workloads in the benchmarked launch configuration with the
    options on; sampled rows against the oracle (a row of a chunk equals a
    one-token step over its own prefix with the same options, pinned on the
    oracle)."""
    wl = W.by_index(idx)
    _log(f"attention softcap={cap} window={win}: {wl.name}")
    d = device_inputs(wl, backend="torch")
    out = run_attention(wl, d, softcap=cap, local_window_size=win)
    assert torch.isfinite(out).all()
    picks = _picks(wl, np.random.default_rng(200 + idx))
    ref, toks = oracle_rows(wl, d, picks, softcap=cap, local_window_size=win)
    err = max_err(out[torch.from_numpy(toks).cuda()], ref)
    _log(f"  {len(picks)} sampled rows, max error {err:.3g}")
    assert err <= TOL[wl.dtype]


FP8_CASES = [
    ("decode W100 cap1", _decode_splits, 1.0, 100),
    ("decode W1500", _decode_splits, 0.0, 1500),
    ("speculative 4 x G4 bf16 W300 cap1.5",
     lambda: W.custom([4, 2, 1, 4], [4, 700, 2049, 3000], 16, 4, 128, 32, dtype="bf16"), 1.5, 300),
]


@pytest.mark.parametrize("name,make,cap,win", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_window_softcap_fp8_small(name, make, cap, win):
    wl = make()
    _log(f"fp8 attention softcap={cap} window={win}: {wl.name}")
    d = device_inputs_fp8(wl)
    out = run_attention_fp8(wl, d, softcap=cap, local_window_size=win)
    assert torch.isfinite(out).all()
    err = max_err(out, oracle_full_fp8(wl, d, softcap=cap, local_window_size=win))
    _log(f"  max error {err:.3g}")
    assert err <= TOL[wl.dtype]


def test_window_softcap_fp8_decode_sampled():
    wl = W.by_index(3)
    _log(f"fp8 attention softcap=1 window=2000: {wl.name}")
    d = device_inputs_fp8(wl, backend="torch")
    out = run_attention_fp8(wl, d, softcap=1.0, local_window_size=2000)
    assert torch.isfinite(out).all()
    picks = _picks(wl, np.random.default_rng(300))
    ref, toks = oracle_rows_fp8(wl, d, picks, softcap=1.0, local_window_size=2000)
    err = max_err(out[torch.from_numpy(toks).cuda()], ref)
    _log(f"  {len(picks)} sampled rows, max error {err:.3g}")
    assert err <= TOL[wl.dtype]
