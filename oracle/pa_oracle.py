"""fp64 CPU oracle for paged-KV-cache scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the library.  It is a
plain, slow, obviously correct statement of what the GPU path computes, in
float64 NumPy, with no blocking, fusion or reordering beyond the definition.

Sources, cited by page and section:

* [PA] onnxruntime pull request #31611, "[WebGPU] Initial PagedAttention
  implementation (1/n)":
  - "Description": new K/V rows are scattered into a paged KV cache, queries
    arrive packed by sequence (continuous batching), and the output is packed
    back to (token_count, hidden_size);
  - "FlashAttention: optional seqlens_q input": each sequence's past length is
    its total KV length minus its own new-query length, never a clamp of
    total minus the batch's longest query (the clamp is the bug the pull
    request fixes);
  - maintainer review, the list of items checked and found correct: the
    token-to-sequence scan picks the first sequence i whose cumulative end
    exceeds the token index (so empty sequences are skipped), the causal
    length of query row q is past + q + 1, the scatter block addressing, and
    the GQA head mapping.
* [FLEX] onnx-light operator documentation, "FlexAttention"
  (ai.onnx.preview):
  - "FlexAttention Computation": scores are Q times K transposed, times
    scale; probabilities are a softmax over the key axis; the output is
    probabilities times V;
  - "Grouped Query Attention (GQA)": query head h reads KV head
    floor(h / group_size) with group_size = q_num_heads / kv_num_heads;
  - "Modifier Subgraphs": masked scores are written as -inf, softmax runs in
    float32 for non-double inputs (here: float64 throughout);
  - examples test_cc_flex_attention_basic and test_cc_flex_attention_gqa
    (the printed outputs are stored under tests/golden/ and pin this file).

Readings where the pages are silent (each is also listed in the design
notes): the paged cache is laid out [num_blocks, block_size, num_kv_heads,
head_size]; ``seqlens_kv[b]`` is the total KV length including this step's
new tokens; the causal mask is bottom-right aligned (key j is visible to new
query row i iff j <= past_b + i); ``scale`` is used exactly as the float32
value that crosses the C ABI, 0 included; a negative slot means "do not
write this token".  The page also names two attention options it leaves
undefined (its v1 rejects them up front, its roadmap lifts them in phase 2):
``softcap`` c > 0 caps each scaled score as c * tanh(s / c) before the mask
and the softmax, and ``local_window_size`` W > 0 limits new row i to its
last W keys, past_b + i - W < j <= past_b + i.

Every function here is pinned by tests in tests/test_oracle_pins.py against
the printed examples, closed forms, invariants and brute force.
"""

from __future__ import annotations

import math

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------
# Core SDPA, as FlexAttention defines it ([FLEX] "FlexAttention Computation").
# ----------------------------------------------------------------------------

def softcap_scores(scores, softcap):
    """The score soft cap: c * tanh(s / c) on the scaled scores for c > 0
    (a score modifier in [FLEX]'s sense; the PagedAttention page names the
    ``softcap`` option without defining it, this is the reading taken);
    c <= 0 leaves the scores unchanged."""
    c = float(np.float32(softcap))
    if c <= 0.0:
        return scores
    return c * np.tanh(scores / c)


def sdpa(q, k, v, scale, visible=None, softcap=0.0):
    """Scaled dot-product attention for one head.

    q: [Sq, D], k: [Skv, D], v: [Skv, Dv]; ``visible``: bool [Sq, Skv] or
    None.  Scores are scaled, soft-capped (``softcap`` > 0), then masked
    scores become -inf before the softmax ([FLEX], masking written as -inf).
    Returns float64 [Sq, Dv].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    scores = softcap_scores((q @ k.T) * float(scale), softcap)
    if visible is not None:
        visible = np.asarray(visible, dtype=bool)
        if not visible.any(axis=-1).all():
            raise ValueError("a query row has no visible key")
        scores = np.where(visible, scores, -np.inf)
    row_max = scores.max(axis=-1, keepdims=True)
    weights = np.exp(scores - row_max)
    probs = weights / weights.sum(axis=-1, keepdims=True)
    return probs @ v


def flex_attention_dense(Q, K, V, scale=None):
    """FlexAttention on rank-4 inputs with no score_mod / prob_mod.

    Q: [B, Hq, Sq, D], K: [B, Hk, Skv, D], V: [B, Hk, Skv, Dv].  Query head h
    uses KV head floor(h / (Hq / Hk)) ([FLEX] "Grouped Query Attention").
    ``scale=None`` means 1/sqrt(head_size): the page prints no default, and
    its two worked examples reproduce with that value only (pinned by tests).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, Hq, Sq, D = Q.shape
    Hk = K.shape[1]
    if Hq % Hk:
        raise ValueError("q_num_heads must be a multiple of kv_num_heads")
    group = Hq // Hk
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    Y = np.zeros((B, Hq, Sq, V.shape[-1]))
    for b in range(B):
        for h in range(Hq):
            kh = h // group
            Y[b, h] = sdpa(Q[b, h], K[b, kh], V[b, kh], scale)
    return Y


# ----------------------------------------------------------------------------
# Paged-cache bookkeeping ([PA] "Description" and the review's checked list).
# ----------------------------------------------------------------------------

def seq_of_token(cu_seqlens_q, t):
    """Sequence owning packed token t: the first b with cu[b+1] > t.

    Zero-length sequences (cu[b+1] == cu[b]) are skipped by construction.
    """
    cu = np.asarray(cu_seqlens_q)
    for b in range(len(cu) - 1):
        if cu[b + 1] > t:
            return b
    raise ValueError(f"token {t} lies beyond cu_seqlens_q[-1]={cu[-1]}")


def slots_from_block_table(cu_seqlens_q, seqlens_kv, block_table, block_size):
    """Cache slot of every new (packed) token, derived from the block table.

    Token t of sequence b sits at KV position pos = past_b + (t - cu[b]) with
    past_b = seqlens_kv[b] - q_len_b; its slot is
    block_table[b][pos // block_size] * block_size + pos % block_size.
    """
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    L = np.asarray(seqlens_kv, dtype=np.int64)
    table = np.asarray(block_table, dtype=np.int64)
    T = int(cu[-1])
    slots = np.empty(T, dtype=np.int64)
    for t in range(T):
        b = seq_of_token(cu, t)
        q_len = cu[b + 1] - cu[b]
        past = L[b] - q_len
        pos = past + (t - cu[b])
        slots[t] = table[b, pos // block_size] * block_size + pos % block_size
    return slots


def scatter_kv(k_new, v_new, slot_mapping, k_cache, v_cache, block_size):
    """Write each new token's K/V row into its cache slot, in place.

    k_new, v_new: [T, Hk, D]; caches: anything indexable as
    cache[block][offset] -> [Hk, D] (an array [NB, bs, Hk, D] or a dict of
    per-block arrays).  A negative slot skips the token.  Pass raw bit
    patterns (e.g. uint16 views) to make the copy bitwise.
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    for t in range(slots.shape[0]):
        s = int(slots[t])
        if s < 0:
            continue
        blk, off = divmod(s, block_size)
        k_cache[blk][off] = k_new[t]
        v_cache[blk][off] = v_new[t]


def gather_sequence(cache, table_row, length, block_size):
    """Walk one sequence's block table: rows 0..length-1 -> [length, Hk, D]."""
    rows = []
    n_blocks = -(-int(length) // block_size)
    for k in range(n_blocks):
        blk = int(table_row[k])
        take = min(block_size, int(length) - k * block_size)
        rows.append(np.asarray(cache[blk])[:take])
    if not rows:
        shape = np.asarray(cache[0]).shape[1:]
        return np.zeros((0,) + tuple(shape))
    return np.concatenate(rows, axis=0)


def _attention_impl(q, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache,
                    scale, num_heads, num_kv_heads, block_size, past_of, softcap=0.0,
                    local_window_size=0):
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    L = np.asarray(seqlens_kv, dtype=np.int64)
    table = np.asarray(block_table)
    B = len(cu) - 1
    T = int(cu[-1])
    if num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    group = num_heads // num_kv_heads
    q = _f64(q)
    if q.ndim == 2:                          # [T, Hq*D] packed rows
        q = q.reshape(T, num_heads, q.shape[1] // num_heads)
    D = q.shape[-1]
    scale = float(np.float32(scale))       # the value that crosses the ABI
    out = np.zeros((T, num_heads, D))
    max_q = int((cu[1:] - cu[:-1]).max()) if B else 0
    for b in range(B):
        q_len = int(cu[b + 1] - cu[b])
        if q_len == 0:
            continue
        past = past_of(int(L[b]), q_len, max_q)
        if past < 0:
            raise ValueError(f"sequence {b}: seqlens_kv < q_len")
        Kb = _f64(gather_sequence(k_cache, table[b], L[b], block_size))
        Vb = _f64(gather_sequence(v_cache, table[b], L[b], block_size))
        i = np.arange(q_len)[:, None]
        j = np.arange(int(L[b]))[None, :]
        visible = j <= past + i                  # causal length past + i + 1
        if local_window_size > 0:                # the last W keys up to the row's own
            visible &= j > past + i - int(local_window_size)
        rows = slice(int(cu[b]), int(cu[b + 1]))
        for h in range(num_heads):
            kh = h // group
            out[rows, h] = sdpa(q[rows, h], Kb[:, kh], Vb[:, kh], scale, visible, softcap)
    return out


def attention(q, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache,
              scale, num_heads, num_kv_heads, block_size, softcap=0.0, local_window_size=0):
    """Paged causal GQA attention over packed variable-length queries.

    q: [T, Hq, D] (or [T, Hq*D]); cu_seqlens_q: [B+1]; seqlens_kv: [B] (total
    KV length including the new tokens); block_table: [B, MB]; caches: see
    ``scatter_kv``.  For each sequence b with q_len_b = cu[b+1]-cu[b] and
    past_b = seqlens_kv[b] - q_len_b, new query row i attends to KV positions
    0..past_b+i, walking the block table.  Returns float64 [T, Hq, D].

    Options the PagedAttention page names without defining (readings taken):
    ``softcap`` c > 0 replaces each scaled score s by c * tanh(s / c) before
    the mask and softmax; ``local_window_size`` W > 0 restricts row i to the
    last W of its keys, past_b + i - W < j <= past_b + i (the row's own key
    included).  0 disables either.
    """
    return _attention_impl(q, cu_seqlens_q, seqlens_kv, block_table, k_cache,
                           v_cache, scale, num_heads, num_kv_heads, block_size,
                           past_of=lambda L, q_len, max_q: L - q_len, softcap=softcap,
                           local_window_size=local_window_size)


def attention_buggy_clamp(q, cu_seqlens_q, seqlens_kv, block_table, k_cache,
                          v_cache, scale, num_heads, num_kv_heads, block_size):
    """The pre-fix behaviour [PA] describes, kept only to show the tests can
    tell it apart: past is clamp(total_kv_b - max_seqlen_q, 0) for every
    sequence instead of total_kv_b - q_len_b."""
    return _attention_impl(q, cu_seqlens_q, seqlens_kv, block_table, k_cache,
                           v_cache, scale, num_heads, num_kv_heads, block_size,
                           past_of=lambda L, q_len, max_q: max(L - max_q, 0))


def attention_loops(q, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache,
                    scale, num_heads, num_kv_heads, block_size, softcap=0.0,
                    local_window_size=0):
    """Pure-Python brute force of ``attention`` for tiny inputs.

    Walks every (token, head, key) with scalar float arithmetic and reads each
    K/V row through block_table[b][j // block_size], offset j % block_size;
    the window is a key range, the soft cap a scalar math.tanh.
    """
    cap = float(np.float32(softcap))
    cu = [int(x) for x in cu_seqlens_q]
    L = [int(x) for x in seqlens_kv]
    T = cu[-1]
    group = num_heads // num_kv_heads
    q = _f64(q)
    if q.ndim == 2:
        q = q.reshape(T, num_heads, q.shape[1] // num_heads)
    D = q.shape[-1]
    scale = float(np.float32(scale))
    out = np.zeros((T, num_heads, D))
    for t in range(T):
        b = seq_of_token(cu, t)
        q_len = cu[b + 1] - cu[b]
        past = L[b] - q_len
        i = t - cu[b]
        j0 = max(0, past + i + 1 - local_window_size) if local_window_size > 0 else 0
        keys = list(range(j0, past + i + 1))
        for h in range(num_heads):
            kh = h // group
            scores = []
            for j in keys:
                blk = int(block_table[b][j // block_size])
                krow = k_cache[blk][j % block_size][kh]
                s = 0.0
                for d in range(D):
                    s += float(q[t, h, d]) * float(krow[d])
                s *= scale
                if cap > 0.0:
                    s = cap * math.tanh(s / cap)
                scores.append(s)
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            tot = sum(w)
            for d in range(D):
                acc = 0.0
                for j, wj in zip(keys, w):
                    blk = int(block_table[b][j // block_size])
                    acc += wj * float(v_cache[blk][j % block_size][kh][d])
                out[t, h, d] = acc / tot
    return out


# ----------------------------------------------------------------------------
# Split-KV: partial softmax state and its log-sum-exp merge.
# ----------------------------------------------------------------------------

def attention_partial(q_rows, k_rows, v_rows, scale, visible):
    """Unnormalised softmax state of query rows over one subset of keys.

    Returns (m, l, acc): m = max visible score (-inf if none), l = sum of
    exp(s - m), acc = sum of exp(s - m) * v, so that acc / l is the attention
    output restricted to the subset.
    """
    s = (_f64(q_rows) @ _f64(k_rows).T) * float(scale)
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=-1) if s.shape[-1] else np.full(s.shape[0], -np.inf)
    base = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(s - base[:, None])
    return m, w.sum(axis=-1), w @ _f64(v_rows)


def combine_partials(parts):
    """Merge (m, l, acc) states of disjoint key subsets into the output:
    M = max m_s; O = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s."""
    M = np.max(np.stack([p[0] for p in parts]), axis=0)
    num = 0.0
    den = 0.0
    for m, l, acc in parts:
        f = np.where(np.isfinite(m), np.exp(m - M), 0.0)
        num = num + f[:, None] * acc
        den = den + f * l
    return num / den[:, None]


# ----------------------------------------------------------------------------
# Metadata preconditions (debug validation of what the kernels trust).
# ----------------------------------------------------------------------------

def validate_metadata(cu_seqlens_q, seqlens_kv, block_table, num_blocks,
                      block_size, num_tokens=None, slot_mapping=None):
    """Return a list of precondition violations (empty when valid)."""
    errs = []
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    L = np.asarray(seqlens_kv, dtype=np.int64)
    table = np.asarray(block_table, dtype=np.int64)
    B = len(cu) - 1
    if B < 0 or cu[0] != 0:
        errs.append("cu_seqlens_q[0] must be 0")
    if np.any(np.diff(cu) < 0):
        errs.append("cu_seqlens_q must be nondecreasing")
    if num_tokens is not None and B >= 0 and cu[-1] != num_tokens:
        errs.append("cu_seqlens_q[num_seqs] must equal num_tokens")
    for b in range(max(B, 0)):
        q_len = cu[b + 1] - cu[b]
        if L[b] < q_len:
            errs.append(f"seq {b}: seqlens_kv < q_len")
        need = -(-int(L[b]) // block_size)
        if need > table.shape[1]:
            errs.append(f"seq {b}: needs {need} blocks > max_blocks_per_seq")
            continue
        used = table[b, :need]
        if np.any((used < 0) | (used >= num_blocks)):
            errs.append(f"seq {b}: block id out of range")
    if slot_mapping is not None:
        s = np.asarray(slot_mapping, dtype=np.int64)
        if np.any(s >= num_blocks * block_size):
            errs.append("slot beyond the cache")
        live = s[s >= 0]
        if np.unique(live).size != live.size:
            errs.append("duplicate non-negative slots")
    return errs
