"""pa_attention_rope (through the C ABI): Q read from the packed QKV rows and
rotated as it is loaded, after pa_rotary_scatter_kv has scattered the
rotated K and plain V without writing Q.

Bars: bitwise equal to the two-step path (pa_rotary_scatter_kv writing the
rotated Q, then pa_attention on it), since both rotate with the same
functions and the attention then sees the same Q bits; the caches the
Q-less scatter leaves are bitwise those of the two-step path; and the fused
output is within the plain attention bars of the fp64 oracle's rotation and
attention.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_pa_amd as pa
from oracle import rotary as R
from paged_kv_cache_pa_amd import workloads as W
from gpu_util import TOL, max_err, nan_cache, require_gpu
from pa_testutil import oracle_caches, to_np64

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _setup(wl, rdim, inter):
    """Device values, packed QKV rows of this step's tokens, rope tables, and
    caches holding every history key rotated at its position (one rotary
    scatter over all positions) and its value."""
    require_gpu()
    vals = W.make_values(wl)
    dev = {k: v.cuda() for k, v in vals.items()}
    rows = torch.from_numpy(wl.new_rows).cuda()
    T = wl.num_tokens
    q, k_new, v_new = dev["q"], dev["k_all"][rows].contiguous(), dev["v_all"][rows].contiguous()
    d = dict(q=q, k_all=dev["k_all"], v_all=dev["v_all"],
             cu=torch.from_numpy(wl.cu_seqlens_q).cuda(),
             lens=torch.from_numpy(wl.seqlens_kv.astype(np.int32)).cuda(),
             table=torch.from_numpy(wl.block_table.astype(np.int32)).cuda(),
             kc=nan_cache(wl), vc=nan_cache(wl))
    d["packed"] = torch.cat([q.reshape(T, -1), k_new.reshape(T, -1), v_new.reshape(T, -1)],
                            dim=1).contiguous()
    cos, sin = W.rope_tables(int(wl.seqlens_kv.max()), rdim, wl.dtype)
    d["cos"], d["sin"] = cos.cuda(), sin.cuda()
    kv_cu = torch.from_numpy(wl.kv_cu.astype(np.int32)).cuda()
    pa.pa_rotary_scatter_kv(None, kv_cu, d["lens"], d["table"], d["kc"], d["vc"], wl.num_heads,
                            wl.num_kv_heads, key=d["k_all"], value=d["v_all"], cos_cache=d["cos"],
                            sin_cache=d["sin"], interleaved=inter, write_q=False)
    torch.cuda.synchronize()
    return d


def _two_step(wl, d, inter, **opts):
    q_rot = pa.pa_rotary_scatter_kv(d["packed"], d["cu"], d["lens"], d["table"], d["kc"], d["vc"],
                                    wl.num_heads, wl.num_kv_heads, cos_cache=d["cos"],
                                    sin_cache=d["sin"], interleaved=inter)
    out = pa.pa_attention(q_rot, d["cu"], d["lens"], d["table"], d["kc"], d["vc"], wl.scale,
                          wl.num_heads, wl.num_kv_heads, **opts)
    torch.cuda.synchronize()
    return out


def _fused(wl, d, inter, **opts):
    assert pa.pa_rotary_scatter_kv(d["packed"], d["cu"], d["lens"], d["table"], d["kc"], d["vc"],
                                   wl.num_heads, wl.num_kv_heads, cos_cache=d["cos"],
                                   sin_cache=d["sin"], interleaved=inter, write_q=False) is None
    out = pa.pa_attention_rope(d["packed"].view(wl.num_tokens, -1, wl.head_size), d["cu"],
                               d["lens"], d["table"], d["kc"], d["vc"], wl.scale, wl.num_heads,
                               wl.num_kv_heads, cos_cache=d["cos"], sin_cache=d["sin"],
                               interleaved=inter, **opts)
    torch.cuda.synchronize()
    return out


CASES = [
    # name, workload, rotary_dim, interleaved, attention options
    ("f16 D128 R128 split G4 decode+prefill",
     lambda: W.custom([5, 1, 64, 1], [40, 1030, 300, 17], 16, 4, 128, 16), 128, False, {}),
    ("f16 D128 R128 interleaved G4 decode+prefill",
     lambda: W.custom([5, 1, 64, 1], [40, 1030, 300, 17], 16, 4, 128, 16), 128, True, {}),
    ("bf16 D128 R64 split G8 cap30 window500",
     lambda: W.custom([1, 2, 100, 1], [5000, 33, 700, 2100], 64, 8, 128, 16, dtype="bf16"), 64,
     False, dict(softcap=30.0, local_window_size=500)),
    ("bf16 D64 R32 interleaved MHA",
     lambda: W.custom([3, 9, 1], [3, 50, 800], 4, 4, 64, 16, dtype="bf16"), 32, True, {}),
    ("f16 D128 R48 split G16 bs64",
     lambda: W.custom([1, 16, 3], [600, 16, 2000], 32, 2, 128, 64), 48, False, {}),
]


@pytest.mark.parametrize("name,make,rdim,inter,opts", CASES, ids=[c[0] for c in CASES])
def test_fused_matches_two_step_bitwise(name, make, rdim, inter, opts):
    wl = make()
    _log(f"fused rope vs two-step: {name}")
    d = _setup(wl, rdim, inter)
    ref = _two_step(wl, d, inter, **opts).clone()
    kc, vc = d["kc"].clone(), d["vc"].clone()
    out = _fused(wl, d, inter, **opts)
    # the Q-less scatter rewrote the same K/V bits
    assert torch.equal(kc.view(torch.int16), d["kc"].view(torch.int16))
    assert torch.equal(vc.view(torch.int16), d["vc"].view(torch.int16))
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_fused_full_size_mixed_batch_bitwise():
    """The large mixed batch (64/8 heads, 8432 new tokens, contexts to 32k),
    split pairing over the whole head, in the launch configuration the
    benchmark times."""
    wl = W.by_index(5)
    _log(f"fused rope vs two-step, full size: {wl.name}")
    d = _setup(wl, wl.head_size, False)
    ref = _two_step(wl, d, False).clone()
    out = _fused(wl, d, False)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("inter", [False, True])
def test_fused_against_oracle(inter):
    """The fused path against the oracle's rotation (rounded to the dtype, as
    the kernels round it) and attention."""
    wl = W.custom([5, 1, 64, 1], [40, 1030, 300, 17], 16, 4, 128, 16)
    _log(f"fused rope vs oracle, interleaved={inter}")
    d = _setup(wl, 96, inter)
    out = _fused(wl, d, inter)
    cos, sin = to_np64(d["cos"]), to_np64(d["sin"])
    rnd = lambda x: to_np64(torch.from_numpy(x).to(torch.float16))  # noqa: E731
    pos_all = np.concatenate([np.arange(L) for L in wl.seqlens_kv])
    k_rot = rnd(R.rotary_embedding(to_np64(d["k_all"]), pos_all, cos, sin, inter))
    q_r = rnd(R.rotary_embedding(to_np64(d["q"]), R.token_positions(wl.cu_seqlens_q,
                                                                     wl.seqlens_kv),
                                 cos, sin, inter))
    kc, vc = oracle_caches(wl, k_rot, to_np64(d["v_all"]))
    ref = oracle.attention(q_r, wl.cu_seqlens_q, wl.seqlens_kv, wl.block_table, kc, vc, wl.scale,
                           wl.num_heads, wl.num_kv_heads, wl.block_size)
    err = max_err(out, ref)
    _log(f"  max error {err:.3g}")
    assert err <= TOL[wl.dtype]


def test_strided_q_without_tables_is_pa_attention():
    """No tables: pa_attention_rope on the packed rows equals pa_attention on
    the contiguous Q, bitwise."""
    wl = W.custom([7, 1, 40], [100, 3000, 40], 32, 8, 128, 16, dtype="bf16")
    _log("strided Q, no rotation")
    d = _setup(wl, 64, False)
    ref = pa.pa_attention(d["q"], d["cu"], d["lens"], d["table"], d["kc"], d["vc"], wl.scale,
                          wl.num_heads, wl.num_kv_heads)
    out = pa.pa_attention_rope(d["packed"].view(wl.num_tokens, -1, wl.head_size), d["cu"],
                               d["lens"], d["table"], d["kc"], d["vc"], wl.scale, wl.num_heads,
                               wl.num_kv_heads)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
