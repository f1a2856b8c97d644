"""Rotary position embedding and the packed-QKV split ahead of the paged
cache: plain CPU statement of what happens to the new tokens before the
attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the library.

Sources, cited by page and section:

* [PA] "[WebGPU] Initial PagedAttention implementation (1/n)": the file
  summaries list a program that splits packed QKV into separate Q, K and V
  and one that applies the rotary embedding to the packed token tensors,
  both ahead of the scatter; the review's summary checks the rotary's
  interleaved and split pairing, its sign, and the pass-through of the
  dimensions at and beyond the rotary dimension.
* The rotation itself is the rotary position embedding of the RoFormer
  paper (Su et al., "RoFormer: Enhanced Transformer with Rotary Position
  Embedding", section 3.2): each pair of dimensions (a, b) of a query or
  key at position p is turned by the angle of that pair at p, i.e. the
  complex number x_a + i x_b is multiplied by cos + i sin.

Readings where the pages are silent (listed in the design notes):

* packed QKV: one row per token holding its num_heads query heads, then its
  num_kv_heads key heads, then its num_kv_heads value heads, head_size
  elements each;
* cos and sin come from caller-supplied tables cos_cache / sin_cache of
  shape [max_position, rotary_dim / 2]; pair k of a row at position p uses
  cos_cache[p][k] and sin_cache[p][k];
* pairing: interleaved pairs are (2k, 2k+1); split pairs are
  (k, k + rotary_dim / 2); k < rotary_dim / 2; dimensions >= rotary_dim
  pass through unchanged;
* rotation: x_a' = x_a cos - x_b sin, x_b' = x_b cos + x_a sin (the sign the
  review checks: minus on the first element of the pair);
* the position of new token i of sequence b is its KV position
  past_b + i (past_b = seqlens_kv[b] - q_len_b), the same position the
  causal mask and the scatter use; Q and K are both rotated, V is not.

Every function here is pinned by tests in tests/test_oracle_rotary_pins.py.
"""

from __future__ import annotations

import numpy as np

from .pa_oracle import scatter_kv, slots_from_block_table


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def token_positions(cu_seqlens_q, seqlens_kv):
    """KV position of every packed new token: past_b + i for token i of
    sequence b."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    L = np.asarray(seqlens_kv, dtype=np.int64)
    pos = np.empty(int(cu[-1]), dtype=np.int64)
    for b in range(len(L)):
        q_len = cu[b + 1] - cu[b]
        pos[cu[b]:cu[b + 1]] = L[b] - q_len + np.arange(q_len)
    return pos


def pair_indices(rotary_dim, interleaved):
    """The (a, b) dimension indices of the rotary_dim / 2 rotated pairs."""
    k = np.arange(rotary_dim // 2)
    if interleaved:
        return 2 * k, 2 * k + 1
    return k, k + rotary_dim // 2


def rotary_embedding(x, positions, cos_cache, sin_cache, interleaved):
    """Rotated copy (float64) of x [T, H, D]: row t of every head turned by
    the angles of position positions[t]; rotary_dim = 2 * cos_cache's
    second extent; dimensions from rotary_dim on are copied."""
    x = _f64(x)
    cos = _f64(cos_cache)[np.asarray(positions)][:, None, :]   # [T, 1, R/2]
    sin = _f64(sin_cache)[np.asarray(positions)][:, None, :]
    a, b = pair_indices(2 * cos.shape[-1], interleaved)
    out = x.copy()
    out[..., a] = x[..., a] * cos - x[..., b] * sin
    out[..., b] = x[..., b] * cos + x[..., a] * sin
    return out


def split_packed_qkv(qkv, num_heads, num_kv_heads):
    """Packed rows [T, (Hq + 2 Hk) * D] (or [T, Hq + 2 Hk, D]) -> views q
    [T, Hq, D], k [T, Hk, D], v [T, Hk, D]."""
    qkv = np.asarray(qkv)
    T = qkv.shape[0]
    x = qkv.reshape(T, num_heads + 2 * num_kv_heads, -1)
    return (x[:, :num_heads], x[:, num_heads:num_heads + num_kv_heads],
            x[:, num_heads + num_kv_heads:])


def rotary_scatter_kv(query, key, value, cos_cache, sin_cache, interleaved, cu_seqlens_q,
                      seqlens_kv, block_table, k_cache, v_cache, block_size, num_heads,
                      num_kv_heads):
    """The steps ahead of the attention for one batch of new tokens:

    1. key None: query holds packed QKV rows, split into Q, K, V;
    2. cos_cache not None: Q and K rotated at each token's position;
    3. K and V written into the paged caches at the slots the block table
       gives each token's position (in place);

    returns Q (rotated or not) as float64 [T, Hq, D].  Positions must lie
    below cos_cache's first extent."""
    if key is None:
        q, k, v = split_packed_qkv(query, num_heads, num_kv_heads)
    else:
        q, k, v = query, key, value
    q, k, v = _f64(q), _f64(k), _f64(v)
    if cos_cache is not None:
        pos = token_positions(cu_seqlens_q, seqlens_kv)
        if len(pos) and pos.max() >= np.asarray(cos_cache).shape[0]:
            raise ValueError("a token position lies beyond the cos/sin tables")
        q = rotary_embedding(q, pos, cos_cache, sin_cache, interleaved)
        k = rotary_embedding(k, pos, cos_cache, sin_cache, interleaved)
    slots = slots_from_block_table(cu_seqlens_q, seqlens_kv, block_table, block_size)
    scatter_kv(k, v, slots, k_cache, v_cache, block_size)
    return q
