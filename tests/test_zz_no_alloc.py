"""pa_attention_noalloc (the library's fixed device scratch instead of a
caller workspace) against pa_attention, through the C ABI.

Two calls in a row on different batches, the second smaller than the first,
so anything the scratch keeps from the first call would show in the second;
then the full pure-decode workload.  Each output is bitwise pa_attention's
output for the same inputs (same kernels and plan), and within the fp16 /
bf16 bars of the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_pa_amd as pa
from paged_kv_cache_pa_amd import workloads as W
from gpu_util import TOL, device_inputs, max_err, oracle_full, run_attention

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _noalloc(wl, d, **kw):
    out = torch.empty_like(d["q"])
    pa.pa_attention_noalloc(d["q"], d["cu"], d["lens"], d["table"], d["kc"], d["vc"], wl.scale,
                            wl.num_heads, wl.num_kv_heads, out, **kw)
    torch.cuda.synchronize()
    return out


def test_noalloc_two_calls_second_smaller():
    big = W.custom([1, 300, 1, 2, 1, 37], [4000, 900, 2500, 1030, 70, 2100], 32, 8, 128, 16,
                   seed=51)
    small = W.custom([1, 5], [1500, 40], 32, 8, 128, 16, dtype="bf16", seed=52)
    for wl in (big, small):
        _log(f"noalloc: {wl.name}")
        d = device_inputs(wl)
        got = _noalloc(wl, d)
        ref = run_attention(wl, d)
        assert torch.equal(got, ref), wl.name
        err = max_err(got, oracle_full(wl, d))
        _log(f"  bitwise pa_attention; oracle max abs error {err:.3g}")
        assert err <= TOL[wl.dtype]


def test_noalloc_options_and_repeat():
    """Soft cap and window through the scratch path, twice in a row."""
    wl = W.custom([1, 70, 1], [3100, 800, 1500], 32, 8, 128, 16, seed=53)
    _log(f"noalloc with cap and window: {wl.name}")
    d = device_inputs(wl)
    opts = dict(softcap=30.0, local_window_size=700)
    a = _noalloc(wl, d, **opts)
    b = _noalloc(wl, d, **opts)
    ref = run_attention(wl, d, **opts)
    assert torch.equal(a, ref) and torch.equal(b, ref)
    assert max_err(a, oracle_full(wl, d, **opts)) <= TOL[wl.dtype]


def test_noalloc_full_decode_workload():
    """The pure-decode workload (256 sequences, contexts up to 8192, 33 MiB of
    workspace) through the scratch: bitwise pa_attention's output."""
    wl = W.by_index(3)
    _log(f"noalloc: {wl.name}")
    d = device_inputs(wl, backend="torch")
    got = _noalloc(wl, d)
    ref = run_attention(wl, d)
    assert torch.isfinite(got).all()
    assert torch.equal(got, ref)


def test_noalloc_rejects_beyond_scratch():
    """Sizes whose workspace exceeds the fixed scratch are refused before
    anything is launched."""
    wl = W.by_index(5)
    # The large mixed batch's sizes (256 sequences, 8432 tokens, 2048-block
    # table rows: 520 MiB of workspace), with valid metadata all the same.
    q_lens = np.full(256, 32, dtype=np.int32)
    q_lens[-1] = 8432 - 32 * 255
    T = int(q_lens.sum())
    q = torch.zeros((T, wl.num_heads, wl.head_size), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((32, wl.block_size, wl.num_kv_heads, wl.head_size), dtype=torch.bfloat16,
                     device="cuda")
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)).cuda()
    lens = torch.from_numpy(q_lens).cuda()
    table = torch.zeros((256, 2048), dtype=torch.int32, device="cuda")
    with pytest.raises(pa.PAError) as e:
        pa.pa_attention_noalloc(q, cu, lens, table, kc, kc, 0.1, wl.num_heads, wl.num_kv_heads,
                                torch.empty_like(q))
    assert e.value.status == 3   # PA_ERR_WORKSPACE_TOO_SMALL


def test_noalloc_under_graph_capture():
    """The entry point captured in a graph (the caller it is for): each of
    three replays equals the eager output bitwise, with eager work between
    replays that includes an allocation-free call on another batch, which
    overwrites the shared scratch the graph's kernels use."""
    wl = W.custom([1, 40, 1, 3], [3000, 500, 20, 2100], 32, 8, 128, 16, seed=54)
    other = W.custom([2, 1, 17], [5000, 70, 900], 32, 8, 128, 16, seed=55)
    _log(f"noalloc under graph capture: {wl.name}")
    d, d2 = device_inputs(wl), device_inputs(other)
    out = torch.empty_like(d["q"])

    def call():
        pa.pa_attention_noalloc(d["q"], d["cu"], d["lens"], d["table"], d["kc"], d["vc"],
                                wl.scale, wl.num_heads, wl.num_kv_heads, out)

    call()
    torch.cuda.synchronize()
    ref = out.clone()
    assert torch.equal(ref, run_attention(wl, d))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    ref2 = run_attention(other, d2)
    for _ in range(3):
        out.zero_()
        assert torch.equal(_noalloc(other, d2), ref2)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
