"""fp8 (e4m3) paged KV cache: plain CPU statement of the quantized cache.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the library.

Sources, cited by page and section:

* [PA] onnxruntime pull request #31611, "[WebGPU] Initial PagedAttention
  implementation (1/n)", "Roadmap": phase 3 brings the quantized KV cache
  (a cache element type T_CACHE apart from the query type), quantized KV
  first; the review's point 2 notes that the v1 rejects KV-cache
  quantization up front.
* The "[WebGPU] Implement SparseAttentionIndexer" pull-request page, file
  summaries of its bundled CUDA PagedAttention change: packed low-bit caches
  with dequantization on read and per-channel scale control.

The pages name the feature but define no format, so the plainest reading is
taken (listed in the design notes):

* element format: 8-bit floating point e4m3 as the Open Compute Project's
  8-bit floating point specification defines it (sign, 4 exponent bits with
  bias 7, 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9; no
  infinities; the all-ones exponent-and-mantissa pattern is NaN, so the
  largest finite magnitude is 1.75 * 2^8 = 448);
* scales: one positive float32 per (KV head, channel) for K and one for V,
  supplied by the caller and applied as a multiplier on read;
* quantization (the scatter): in float32, y = x * (1 / scale) with the
  reciprocal and the product each rounded to float32; magnitudes above 448
  (infinities included) saturate to 448; y is then rounded to the nearest
  e4m3 value, ties to the even mantissa; a NaN gives code 0xFF;
* dequantization (attention): element value = e4m3 value * scale.
  Attention is then exactly the 16-bit path's attention over the
  dequantized K and V (float64 here).

Every function here is pinned by tests in tests/test_oracle_fp8_pins.py.
"""

from __future__ import annotations

import numpy as np

from .pa_oracle import attention as _attention

E4M3_MAX = 448.0
E4M3_NAN = 0xFF


def e4m3_decode(codes):
    """Value of each e4m3 code (float64; NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0 ** -9
    val = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_encode(y):
    """Code of each float32 value: saturate above 448, then round to the
    nearest e4m3 value with ties to the even mantissa (NaN -> 0xFF)."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)   # exact
    nan = np.isnan(y)
    neg = np.signbit(y)
    a = np.minimum(np.abs(np.where(nan, 0.0, y)), E4M3_MAX)
    # Spacing of the e4m3 grid at a: 2^(e-3) in binade [2^e, 2^(e+1)) for
    # e >= -6; the subnormal range [0, 2^-6) has spacing 2^-9.
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6.0, 8.0)
    step = np.exp2(e - 3.0)
    q = np.rint(a / step) * step            # a / step is exact; rint ties to even
    q = np.minimum(q, E4M3_MAX)
    # Code of the grid value q.
    with np.errstate(divide="ignore"):
        qe = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    is_sub = q < 2.0 ** -6
    mant_sub = np.rint(q / 2.0 ** -9)
    exp_f = np.where(is_sub, 0.0, qe + 7.0)
    mant_n = np.rint((q / np.exp2(qe) - 1.0) * 8.0)
    code = np.where(is_sub, mant_sub, exp_f * 8.0 + mant_n).astype(np.int64)
    code = code | np.where(neg, 0x80, 0)
    code = np.where(nan, E4M3_NAN, code)
    return code.astype(np.uint8)


def quantize(x, scale):
    """Codes of x under per-channel scales (broadcast over the last axes):
    e4m3_encode(float32(x) * float32(1 / scale))."""
    x32 = np.asarray(x, dtype=np.float32)
    s32 = np.asarray(scale, dtype=np.float32)
    inv = (np.float32(1.0) / s32).astype(np.float32)
    y = (x32 * inv).astype(np.float32)
    return e4m3_encode(y)


def dequantize(codes, scale):
    """float64 value of each cached element: e4m3 value times its scale."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float32).astype(np.float64)


def scatter_kv_fp8(k_new, v_new, slot_mapping, k_scale, v_scale, k_cache, v_cache,
                   block_size):
    """The scatter step into fp8 caches of codes [NB, bs, Hk, D]: each token
    with a non-negative slot s writes quantize(row, scale) at
    cache[s // bs][s % bs]; the caches are updated in place."""
    kq = quantize(k_new, k_scale)
    vq = quantize(v_new, v_scale)
    for t, s in enumerate(np.asarray(slot_mapping)):
        s = int(s)
        if s < 0:
            continue
        k_cache[s // block_size, s % block_size] = kq[t]
        v_cache[s // block_size, s % block_size] = vq[t]
    return k_cache, v_cache


class DequantizedCache:
    """Read-only view of an fp8 code cache (an array [NB, bs, Hk, D] or a
    dict of blocks) whose block ``i`` is ``dequantize(codes[i], scale)``."""

    def __init__(self, codes, scale):
        self.codes = codes
        self.scale = np.asarray(scale, dtype=np.float32)

    def __getitem__(self, i):
        return dequantize(np.asarray(self.codes[i]), self.scale)


def attention_fp8(q, cu_seqlens_q, seqlens_kv, block_table, k_codes, v_codes, k_scale,
                  v_scale, scale, num_heads, num_kv_heads, block_size, softcap=0.0,
                  local_window_size=0):
    """Paged attention over fp8 caches: the 16-bit path's attention over the
    dequantized K and V (blocks dequantized as the block table is walked),
    with the same score options."""
    return _attention(q, cu_seqlens_q, seqlens_kv, block_table,
                      DequantizedCache(k_codes, k_scale), DequantizedCache(v_codes, v_scale),
                      scale, num_heads, num_kv_heads, block_size, softcap=softcap,
                      local_window_size=local_window_size)
