"""Seeded synthetic workloads for paged-KV-cache attention.

This module only *makes inputs*: sequence lengths, a block allocation (block
table plus the cache slot of every KV position, as a serving system's block
manager would hand them out) and random Q/K/V values.  It holds none of the
attention arithmetic and is shared, as the one common module, by the tests,
the bench and the oracle-side checks.

Draw order with ``numpy.random.default_rng(seed)``: lengths, then the block
permutation, then values (Q, K, V).  Values are drawn in float64 and rounded
to the storage dtype with round-to-nearest-even; the large workloads draw
their values on the device with ``torch`` (float32 draws, then rounded) so
that multi-GB caches are generated in milliseconds.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f16", "bf16")


@dataclass
class Workload:
    name: str
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    q_lens: np.ndarray          # int32 [B]
    seqlens_kv: np.ndarray      # int32 [B], total KV length incl. new tokens
    block_table: np.ndarray     # int32 [B, MB], -1 where unused
    scale: float
    dist: str                   # "uniform" (U(-1,1)) or "normal" (N(0,1))
    seed: int
    rng_state: dict = field(default=None, repr=False)

    @property
    def num_seqs(self) -> int:
        return int(self.q_lens.shape[0])

    @property
    def cu_seqlens_q(self) -> np.ndarray:
        cu = np.zeros(self.num_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.q_lens)
        return cu

    @property
    def num_tokens(self) -> int:
        return int(self.q_lens.sum())

    @property
    def kv_cu(self) -> np.ndarray:
        """Row offsets of each sequence in the all-positions K/V tensors."""
        cu = np.zeros(self.num_seqs + 1, dtype=np.int64)
        cu[1:] = np.cumsum(self.seqlens_kv.astype(np.int64))
        return cu

    @property
    def kv_slots(self) -> np.ndarray:
        """Cache slot of every KV position of every sequence (int32 [sum L]).

        The allocator gives sequence b the blocks block_table[b][0..]; its
        positions fill them in order, block_size slots per block.
        """
        bs = self.block_size
        out = np.empty(int(self.seqlens_kv.sum()), dtype=np.int64)
        start = 0
        for b in range(self.num_seqs):
            n = int(self.seqlens_kv[b])
            nb = -(-n // bs)
            blocks = self.block_table[b, :nb].astype(np.int64)
            per_block = blocks[:, None] * bs + np.arange(bs, dtype=np.int64)[None, :]
            out[start:start + n] = per_block.reshape(-1)[:n]
            start += n
        return out.astype(np.int32)

    @property
    def new_rows(self) -> np.ndarray:
        """Rows of the all-positions K/V tensors that are this step's new
        tokens (the last q_len_b positions of each sequence), packed order."""
        kv_cu = self.kv_cu
        rows = [np.arange(kv_cu[b + 1] - self.q_lens[b], kv_cu[b + 1], dtype=np.int64)
                for b in range(self.num_seqs)]
        return np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)

    @property
    def slot_mapping(self) -> np.ndarray:
        return self.kv_slots[self.new_rows]


def _allocate(rng, seqlens_kv, block_size, num_blocks, max_blocks_per_seq):
    """Blocks are taken in order from one seeded permutation of the pool."""
    perm = rng.permutation(num_blocks)
    B = len(seqlens_kv)
    table = np.full((B, max_blocks_per_seq), -1, dtype=np.int32)
    nxt = 0
    for b in range(B):
        nb = -(-int(seqlens_kv[b]) // block_size)
        if nb > max_blocks_per_seq or nxt + nb > num_blocks:
            raise ValueError("pool or block-table row too small")
        table[b, :nb] = perm[nxt:nxt + nb]
        nxt += nb
    return table


def _finish(name, rng, dtype, hq, hk, d, bs, nb, mb, q_lens, lens, dist, seed):
    table = _allocate(rng, lens, bs, nb, mb)
    return Workload(name=name, dtype=dtype, num_heads=hq, num_kv_heads=hk,
                    head_size=d, block_size=bs, num_blocks=nb,
                    max_blocks_per_seq=mb,
                    q_lens=np.asarray(q_lens, dtype=np.int32),
                    seqlens_kv=np.asarray(lens, dtype=np.int32),
                    block_table=table, scale=1.0 / math.sqrt(d), dist=dist,
                    seed=seed, rng_state=rng.bit_generator.state)


def tiny(seed=1235):
    """2 sequences, q_len {1,4}, past {28,12}; 4/2 heads, D 64, bs 16, pool 8."""
    rng = np.random.default_rng(seed)
    q_lens = [1, 4]
    lens = [28 + 1, 12 + 4]
    return _finish("tiny mixed: q_len {1,4}, past {28,12}, Hq 4 / Hk 2, D 64, bs 16, fp16",
                   rng, "f16", 4, 2, 64, 16, 8, 2, q_lens, lens, "uniform", seed)


def small(q_lens, seqlens_kv, num_heads, num_kv_heads, seed=1236, dtype="f16"):
    """One case of the small matrix: D 64, bs 256, pool of 4 blocks."""
    rng = np.random.default_rng(seed)
    name = (f"small: q_len {list(q_lens)}, total_kv {list(seqlens_kv)}, "
            f"Hq {num_heads} / Hk {num_kv_heads}, D 64, bs 256, {dtype}")
    return _finish(name, rng, dtype, num_heads, num_kv_heads, 64, 256, 4, 1,
                   q_lens, seqlens_kv, "uniform", seed)


def small_cases():
    """The small matrix: (q0,q1) in {1,4,16}^2, (L0,L1) in {32,64}^2, heads
    8/8 and 8/2 (72 two-sequence cases) plus 12 single-sequence cases."""
    cases = []
    qs, ls = (1, 4, 16), (32, 64)
    for hq, hk in ((8, 8), (8, 2)):
        for q0 in qs:
            for q1 in qs:
                for l0 in ls:
                    for l1 in ls:
                        cases.append(((q0, q1), (l0, l1), hq, hk))
        for q0 in qs:
            for l0 in ls:
                cases.append(((q0,), (l0,), hq, hk))
    return cases


def decode(seed=1237, num_seqs=256):
    """Pure decode: q_len 1, context U{1024..8192}; 32/8 heads, D 128, bs 16,
    pool of 131250 blocks (2.1M tokens), K/V (and Q) N(0,1)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1024, 8192, size=num_seqs, endpoint=True)
    return _finish(f"pure decode: {num_seqs} x q_len 1, context U[1024,8192], Hq 32 / Hk 8, "
                   "D 128, bs 16, fp16", rng, "f16", 32, 8, 128, 16, 131250, 512,
                   np.ones(num_seqs, dtype=np.int32), lens, "normal", seed)


def prefill(seed=1238, num_seqs=8):
    """Chunked prefill: q_len 2048, past U{0..4096}; 32/8 heads, D 128, bs 256."""
    rng = np.random.default_rng(seed)
    past = rng.integers(0, 4096, size=num_seqs, endpoint=True)
    q_lens = np.full(num_seqs, 2048, dtype=np.int32)
    return _finish(f"chunked prefill: {num_seqs} x q_len 2048, past U[0,4096], Hq 32 / Hk 8, "
                   "D 128, bs 256, fp16", rng, "f16", 32, 8, 128, 256, 192, 24,
                   q_lens, past + q_lens, "uniform", seed)


def mixed(seed=1239, n_prefill=16, n_decode=240):
    """Large mixed continuous batch (bf16): 16 prefill chunks of 512 (past
    U{0..8192}) plus 240 decodes (context log-uniform in [1k, 32k]), kinds
    interleaved by a seeded shuffle; 64/8 heads, D 128, bs 16, fragmented
    random block table over a 500224-block pool."""
    rng = np.random.default_rng(seed)
    past = rng.integers(0, 8192, size=n_prefill, endpoint=True)
    ctx = np.exp(rng.uniform(math.log(1024), math.log(32768), size=n_decode))
    ctx = np.clip(np.round(ctx), 1024, 32768).astype(np.int64)
    q_lens = np.concatenate([np.full(n_prefill, 512), np.ones(n_decode)]).astype(np.int32)
    lens = np.concatenate([past + 512, ctx]).astype(np.int64)
    order = rng.permutation(n_prefill + n_decode)
    return _finish(f"large mixed: {n_prefill} x q_len 512 prefill (past U[0,8192]) + "
                   f"{n_decode} decodes (context log-U[1k,32k]), Hq 64 / Hk 8, D 128, bs 16, bf16",
                   rng, "bf16", 64, 8, 128, 16, 500224, 2048,
                   q_lens[order], lens[order], "uniform", seed)


def custom(q_lens, seqlens_kv, num_heads, num_kv_heads, head_size=128, block_size=16,
           dtype="f16", spare_blocks=3, seed=7, dist="uniform", max_blocks_per_seq=None):
    """An arbitrary batch for edge cases: given lengths, a pool with a few
    spare (never referenced) blocks, blocks dealt from a seeded permutation."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(seqlens_kv, dtype=np.int64)
    need = -(-lens // block_size)
    mb = max_blocks_per_seq or max(1, int(need.max()) if len(need) else 1)
    nb = int(need.sum()) + spare_blocks
    name = (f"custom: q_len {list(q_lens)}, total_kv {list(seqlens_kv)}, Hq {num_heads} / "
            f"Hk {num_kv_heads}, D {head_size}, bs {block_size}, {dtype}")
    return _finish(name, rng, dtype, num_heads, num_kv_heads, head_size, block_size, nb, mb,
                   q_lens, lens, dist, seed)


def by_index(i):
    """Workloads 1..5 (the small matrix is 2; its first GQA case stands in)."""
    if i == 1:
        return tiny()
    if i == 2:
        return small((4, 16), (32, 64), 8, 2)
    if i == 3:
        return decode()
    if i == 4:
        return prefill()
    if i == 5:
        return mixed()
    raise ValueError(i)


# ----------------------------------------------------------------------------
# Values
# ----------------------------------------------------------------------------

def torch_dtype(wl):
    import torch
    return torch.float16 if wl.dtype == "f16" else torch.bfloat16


def make_values(wl, device="cpu", backend="numpy"):
    """Random Q [T, Hq, D] and all-positions K, V [sum L, Hk, D] tensors.

    backend "numpy": float64 draws from the workload's own rng stream (after
    the lengths and the block permutation), rounded to the dtype;
    backend "torch": float32 draws from a torch generator seeded with the
    workload seed on ``device`` (for multi-GB workloads).
    """
    import torch
    dt = torch_dtype(wl)
    T, hq, hk, d = wl.num_tokens, wl.num_heads, wl.num_kv_heads, wl.head_size
    n_kv = int(wl.seqlens_kv.sum())
    shapes = ((T, hq, d), (n_kv, hk, d), (n_kv, hk, d))
    out = []
    if backend == "numpy":
        rng = np.random.default_rng()
        rng.bit_generator.state = wl.rng_state
        for shp in shapes:
            x = (rng.uniform(-1.0, 1.0, size=shp) if wl.dist == "uniform"
                 else rng.standard_normal(size=shp))
            out.append(torch.from_numpy(x).to(dt).to(device))
    elif backend == "torch":
        g = torch.Generator(device=device)
        g.manual_seed(int(wl.seed))
        for shp in shapes:
            if wl.dist == "uniform":
                x = torch.rand(shp, generator=g, device=device, dtype=torch.float32)
                x.mul_(2.0).sub_(1.0)
            else:
                x = torch.randn(shp, generator=g, device=device, dtype=torch.float32)
            out.append(x.to(dt))
            del x
    else:
        raise ValueError(backend)
    return {"q": out[0], "k_all": out[1], "v_all": out[2]}


def rope_tables(max_position, rotary_dim, dtype="f16", base=10000.0):
    """cos / sin tables [max_position, rotary_dim / 2] a caller of the rotary
    scatter supplies: the usual rotary frequencies, angle p * base^(-2k / R)
    for pair k at position p, rounded to the dtype (torch CPU tensors)."""
    import torch
    k = np.arange(rotary_dim // 2, dtype=np.float64)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * base ** (-2.0 * k / rotary_dim)
    dt = torch.float16 if dtype == "f16" else torch.bfloat16
    return torch.from_numpy(np.cos(ang)).to(dt), torch.from_numpy(np.sin(ang)).to(dt)


def fp8_scales(wl, seed=None):
    """Per-(KV head, channel) float32 scales of fp8 (e4m3) caches for the
    workload's K and V: c * (1 + 0.5 u), u ~ U[0, 1) from a seeded stream,
    with c = bound / 448 for the value range (bound 1.25 for U(-1,1) values,
    4.5 for N(0,1)), so values within the bound never saturate.  Returns
    numpy (k_scale, v_scale), each [num_kv_heads, head_size]."""
    rng = np.random.default_rng(int(wl.seed) + 7919 if seed is None else seed)
    bound = 1.25 if wl.dist == "uniform" else 4.5
    c = bound / 448.0
    shape = (wl.num_kv_heads, wl.head_size)
    ks = (c * (1.0 + 0.5 * rng.uniform(0.0, 1.0, size=shape))).astype(np.float32)
    vs = (c * (1.0 + 0.5 * rng.uniform(0.0, 1.0, size=shape))).astype(np.float32)
    return ks, vs
