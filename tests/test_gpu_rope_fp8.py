"""pa_rotary_scatter_kv_fp8 (through the C ABI): the rotary step into fp8
(e4m3) caches with per-channel scales.

Bars: the cache codes and the rotated Q are bitwise those of the two-step
path (pa_rotary_scatter_kv into 16-bit caches, then pa_scatter_kv_fp8 of the
rotated rows); the codes equal the oracle's quantization (oracle/kv_fp8.py)
of the kernel's 16-bit rotated rows, bit for bit (the rotation itself is
pinned to the oracle within one ulp by the 16-bit rotary tests); and
attention over caches filled this way is within the fp8 attention bars of
the oracle's fp8 attention.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_pa_amd as pa
from oracle import kv_fp8
from paged_kv_cache_pa_amd import workloads as W
from gpu_util import FP8_NAN, TOL, max_err, nan_cache, require_gpu
from pa_testutil import to_np64

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _codes(wl):
    shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_size)
    return (torch.full(shape, FP8_NAN, dtype=torch.uint8, device="cuda"),
            torch.full(shape, FP8_NAN, dtype=torch.uint8, device="cuda"))


def _setup(wl, rdim):
    require_gpu()
    vals = W.make_values(wl)
    dev = {k: v.cuda() for k, v in vals.items()}
    rows = torch.from_numpy(wl.new_rows).cuda()
    T = wl.num_tokens
    d = dict(q=dev["q"], k_all=dev["k_all"], v_all=dev["v_all"],
             k_new=dev["k_all"][rows].contiguous(), v_new=dev["v_all"][rows].contiguous(),
             cu=torch.from_numpy(wl.cu_seqlens_q).cuda(),
             lens=torch.from_numpy(wl.seqlens_kv.astype(np.int32)).cuda(),
             table=torch.from_numpy(wl.block_table.astype(np.int32)).cuda(),
             slots=torch.from_numpy(wl.slot_mapping.astype(np.int32)).cuda())
    d["packed"] = torch.cat([d["q"].reshape(T, -1), d["k_new"].reshape(T, -1),
                             d["v_new"].reshape(T, -1)], dim=1).contiguous()
    cos, sin = W.rope_tables(int(wl.seqlens_kv.max()), rdim, wl.dtype)
    d["cos"], d["sin"] = cos.cuda(), sin.cuda()
    ks, vs = W.fp8_scales(wl)
    d["ks_np"], d["vs_np"] = ks, vs
    d["ks"], d["vs"] = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
    return d


CASES = [
    ("f16 D128 R128 split G4 packed", lambda: W.custom([5, 1, 33], [40, 17, 100], 16, 4, 128, 16),
     128, False, True),
    ("bf16 D128 R64 interleaved G8 bs32", lambda: W.custom([7, 1, 20], [300, 1025, 20], 16, 2,
                                                           128, 32, dtype="bf16"), 64, True, False),
    ("f16 D64 R48 split MHA packed", lambda: W.custom([3, 9, 1], [3, 50, 800], 4, 4, 64, 16), 48,
     False, True),
]


@pytest.mark.parametrize("name,make,rdim,inter,packed", CASES, ids=[c[0] for c in CASES])
def test_rotary_fp8_matches_two_step_and_oracle_codes(name, make, rdim, inter, packed):
    wl = make()
    _log(f"rotary into fp8 caches: {name}")
    d = _setup(wl, rdim)
    kw = dict(cos_cache=d["cos"], sin_cache=d["sin"], interleaved=inter)
    src = dict(query=d["packed"]) if packed else dict(query=d["q"], key=d["k_new"],
                                                       value=d["v_new"])
    # two-step: rotate into 16-bit caches, then quantize the rotated rows
    k16, v16 = nan_cache(wl), nan_cache(wl)
    q_a = pa.pa_rotary_scatter_kv(cu_seqlens_q=d["cu"], seqlens_kv=d["lens"],
                                  block_table=d["table"], k_cache=k16, v_cache=v16,
                                  num_heads=wl.num_heads, num_kv_heads=wl.num_kv_heads, **src, **kw)
    sl = d["slots"].long()
    k_rot = k16.view(-1, wl.num_kv_heads, wl.head_size)[sl].contiguous()
    v_rows = v16.view(-1, wl.num_kv_heads, wl.head_size)[sl].contiguous()
    kc_a, vc_a = _codes(wl)
    pa.pa_scatter_kv_fp8(k_rot, v_rows, d["slots"], d["ks"], d["vs"], kc_a, vc_a)
    # fused
    kc_b, vc_b = _codes(wl)
    q_b = pa.pa_rotary_scatter_kv_fp8(cu_seqlens_q=d["cu"], seqlens_kv=d["lens"],
                                      block_table=d["table"], k_scale=d["ks"], v_scale=d["vs"],
                                      k_cache=kc_b, v_cache=vc_b, num_heads=wl.num_heads,
                                      num_kv_heads=wl.num_kv_heads, **src, **kw)
    torch.cuda.synchronize()
    assert torch.equal(kc_a, kc_b) and torch.equal(vc_a, vc_b)
    assert torch.equal(q_a.view(torch.int16), q_b.view(torch.int16))
    # the codes are the oracle's quantization of the kernel's rotated rows
    kq = kv_fp8.quantize(k_rot.float().cpu().numpy(), d["ks_np"])
    vq = kv_fp8.quantize(v_rows.float().cpu().numpy(), d["vs_np"])
    np.testing.assert_array_equal(kc_b.view(-1, wl.num_kv_heads, wl.head_size)[sl].cpu().numpy(), kq)
    np.testing.assert_array_equal(vc_b.view(-1, wl.num_kv_heads, wl.head_size)[sl].cpu().numpy(), vq)
    # slots the step does not own keep their NaN codes
    owned = torch.zeros(kc_b.view(-1, wl.num_kv_heads, wl.head_size).shape[0], dtype=torch.bool,
                        device="cuda")
    owned[sl] = True
    assert (kc_b.view(-1, wl.num_kv_heads, wl.head_size)[~owned] == FP8_NAN).all()


@pytest.mark.parametrize("inter", [False, True])
def test_rotary_fp8_attention_end_to_end(inter):
    """History keys rotated into the fp8 caches (a K/V-only call over every
    position, no query), this step's tokens rotated and scattered, then
    pa_attention_fp8 on the rotated Q: against the oracle's fp8 attention
    over the same codes."""
    wl = W.custom([1, 1, 4, 1], [40, 1030, 300, 17], 16, 4, 128, 16)
    _log(f"rotary fp8 end to end, interleaved={inter}")
    d = _setup(wl, 128)
    kc, vc = _codes(wl)
    kv_cu = torch.from_numpy(wl.kv_cu.astype(np.int32)).cuda()
    assert pa.pa_rotary_scatter_kv_fp8(None, kv_cu, d["lens"], d["table"], d["ks"], d["vs"], kc,
                                       vc, wl.num_heads, wl.num_kv_heads, key=d["k_all"],
                                       value=d["v_all"], cos_cache=d["cos"], sin_cache=d["sin"],
                                       interleaved=inter, write_q=False) is None
    q_rot = pa.pa_rotary_scatter_kv_fp8(d["packed"], d["cu"], d["lens"], d["table"], d["ks"],
                                        d["vs"], kc, vc, wl.num_heads, wl.num_kv_heads,
                                        cos_cache=d["cos"], sin_cache=d["sin"], interleaved=inter)
    out = pa.pa_attention_fp8(q_rot, d["cu"], d["lens"], d["table"], kc, vc, d["ks"], d["vs"],
                              wl.scale, wl.num_heads, wl.num_kv_heads, int(wl.q_lens.max()))
    torch.cuda.synchronize()
    ref = kv_fp8.attention_fp8(to_np64(q_rot), wl.cu_seqlens_q, wl.seqlens_kv, wl.block_table,
                               kc.cpu().numpy(), vc.cpu().numpy(), d["ks_np"], d["vs_np"],
                               wl.scale, wl.num_heads, wl.num_kv_heads, wl.block_size)
    err = max_err(out, ref)
    _log(f"  max error {err:.3g}")
    assert torch.isfinite(out).all()
    assert err <= TOL[wl.dtype]
