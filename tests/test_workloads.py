"""The seeded synthetic workloads: shapes, ranges and determinism."""
import numpy as np

from paged_kv_cache_pa_amd import workloads as W


def _blocks_unique(wl):
    used = np.concatenate([wl.block_table[b, : -(-int(wl.seqlens_kv[b]) // wl.block_size)]
                           for b in range(wl.num_seqs)])
    return np.unique(used).size == used.size and used.min() >= 0 and used.max() < wl.num_blocks


def test_tiny_shapes():
    wl = W.tiny()
    vals = W.make_values(wl)
    assert tuple(vals["q"].reshape(wl.num_tokens, -1).shape) == (5, 256)
    assert list(wl.seqlens_kv - wl.q_lens) == [28, 12]
    assert wl.num_blocks == 8 and wl.max_blocks_per_seq == 2
    assert (wl.block_table[0] >= 0).sum() == 2 and (wl.block_table[1] >= 0).sum() == 1
    assert _blocks_unique(wl)


def test_small_matrix_size():
    cases = W.small_cases()
    assert len(cases) == 84
    assert sum(1 for c in cases if len(c[0]) == 2) == 72


def test_determinism():
    a, b = W.tiny(), W.tiny()
    assert np.array_equal(a.block_table, b.block_table)
    va, vb = W.make_values(a), W.make_values(b)
    for n in ("q", "k_all", "v_all"):
        assert bool((va[n] == vb[n]).all())


def test_decode_workload():
    wl = W.decode()
    assert wl.num_seqs == 256 and wl.num_blocks == 131250 and wl.max_blocks_per_seq == 512
    assert wl.seqlens_kv.min() >= 1024 and wl.seqlens_kv.max() <= 8192
    assert (wl.q_lens == 1).all() and _blocks_unique(wl)
    assert wl.num_blocks * wl.block_size * wl.num_kv_heads * wl.head_size > 2**31


def test_prefill_workload():
    wl = W.prefill()
    assert wl.num_seqs == 8 and (wl.q_lens == 2048).all()
    past = wl.seqlens_kv - wl.q_lens
    assert past.min() >= 0 and past.max() <= 4096 and _blocks_unique(wl)


def test_mixed_workload():
    wl = W.mixed()
    assert wl.dtype == "bf16" and wl.num_seqs == 256
    pre = wl.q_lens == 512
    assert pre.sum() == 16 and (wl.q_lens[~pre] == 1).all()
    assert wl.seqlens_kv[~pre].min() >= 1024 and wl.seqlens_kv[~pre].max() <= 32768
    assert (wl.seqlens_kv[pre] - 512).max() <= 8192
    # the kinds interleave rather than sit in two runs
    assert np.count_nonzero(np.diff(pre.astype(int))) > 4
    assert _blocks_unique(wl)
