"""Helpers shared by the tests: golden-file loading and oracle-side inputs.

Oracle-side caches are filled by the oracle's own scatter from the seeded
generator's values; nothing here reads GPU results.
"""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    """Parse a golden file: '# ...' comments, then 'NAME d0 d1 ..' header
    lines each followed by one line of row-major values."""
    lines = [ln for ln in open(os.path.join(GOLDEN, name)) if ln.strip() and not ln.startswith("#")]
    out = {}
    for i in range(0, len(lines), 2):
        head = lines[i].split()
        shape = tuple(int(x) for x in head[1:])
        out[head[0]] = np.array([float(x) for x in lines[i + 1].split()]).reshape(shape)
    return out


def to_np64(t):
    """torch tensor (fp16/bf16/any) -> float64 numpy, exactly."""
    return t.detach().cpu().float().numpy().astype(np.float64)


def oracle_caches(wl, k_all, v_all, fill=np.nan):
    """Oracle-side paged caches [NB, bs, Hk, D] (float64, unused slots
    ``fill``) filled by the oracle's own scatter of the all-positions values
    k_all/v_all [sum L, Hk, D] at the workload's slots."""
    from oracle import scatter_kv
    shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_size)
    kc = np.full(shape, fill)
    vc = np.full(shape, fill)
    scatter_kv(k_all, v_all, wl.kv_slots, kc, vc, wl.block_size)
    return kc, vc


def oracle_caches_for(wl, seqs, k_rows, v_rows, fill=np.nan):
    """Dict-of-blocks oracle caches holding only the blocks of sequences
    ``seqs``; k_rows(b)/v_rows(b) return that sequence's all-positions
    values as float64 [L_b, Hk, D].  Used for sampled checks of multi-GB
    workloads."""
    from oracle import scatter_kv
    shape = (wl.block_size, wl.num_kv_heads, wl.head_size)
    kc, vc = {}, {}
    slots_all = wl.kv_slots
    kv_cu = wl.kv_cu
    for b in seqs:
        n = int(wl.seqlens_kv[b])
        nb = -(-n // wl.block_size)
        for blk in wl.block_table[b, :nb]:
            kc.setdefault(int(blk), np.full(shape, fill))
            vc.setdefault(int(blk), np.full(shape, fill))
        scatter_kv(k_rows(b), v_rows(b), slots_all[kv_cu[b]:kv_cu[b + 1]], kc, vc,
                   wl.block_size)
    return kc, vc


def embed_flex_example(g, pad_to=None):
    """Embed a FlexAttention example (batch 1, no mask) in the paged layout:
    every query row becomes its own sequence with q_len 1 and total KV
    length kv_len, so the causal mask admits every key; all sequences share
    the same physical block(s).  Returns a dict of oracle/GPU inputs and the
    expected output in packed [T, Hq, D] order."""
    Q, K, V, Y = g["Q"][0], g["K"][0], g["V"][0], g["Y"][0]   # [H, S, D]
    hq, sq, d = Q.shape
    hk, skv, _ = K.shape
    D = pad_to or d
    bs = 16
    nb_needed = -(-skv // bs)
    num_blocks = nb_needed + 1
    q = np.zeros((sq, hq, D))
    q[:, :, :d] = Q.transpose(1, 0, 2)
    k_cache = np.full((num_blocks, bs, hk, D), np.nan)
    v_cache = np.full((num_blocks, bs, hk, D), np.nan)
    phys = np.arange(1, num_blocks)          # block 0 stays unused (NaN)
    for j in range(skv):
        k_cache[phys[j // bs], j % bs] = 0.0
        v_cache[phys[j // bs], j % bs] = 0.0
        k_cache[phys[j // bs], j % bs, :, :d] = K[:, j, :]
        v_cache[phys[j // bs], j % bs, :, :d] = V[:, j, :]
    y = np.zeros((sq, hq, D))
    y[:, :, :d] = Y.transpose(1, 0, 2)
    return dict(q=q, cu=np.arange(sq + 1, dtype=np.int32),
                seqlens_kv=np.full(sq, skv, dtype=np.int32),
                block_table=np.tile(phys[None, :nb_needed], (sq, 1)).astype(np.int32),
                k_cache=k_cache, v_cache=v_cache, num_heads=hq, num_kv_heads=hk,
                block_size=bs, num_blocks=num_blocks, scale=1.0 / np.sqrt(d), y=y, d=d)
