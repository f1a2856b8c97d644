"""The C-ABI library on the CPU: it loads, exports every symbol include/pa.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

from paged_kv_cache_pa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libpa.so is not built (python -m paged_kv_cache_pa_amd.build)")
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    syms = _declared_symbols()
    assert set(syms) == set(_lib.EXPORTS)
    for s in syms:
        assert getattr(L, s) is not None


def test_status_strings(L):
    assert L.pa_status_string(0) == b"PA_OK"
    assert L.pa_status_string(2) == b"PA_ERR_NOT_IMPLEMENTED"
    assert L.pa_status_string(99) == b"PA_ERR_UNKNOWN"


def test_workspace_size(L):
    n = L.pa_attention_workspace_size(256, 256, 512, 32, 8, 128, 16)
    assert n > 0 and n % 256 == 0
    assert L.pa_attention_workspace_size(2, 5, 2, 4, 3, 64, 16) == 0      # Hq % Hk
    assert L.pa_attention_workspace_size(2, 5, 2, 4, 2, 96, 16) == 0      # head size
    assert L.pa_attention_workspace_size(2, 5, 2, 4, 2, 64, 24) == 0      # block size


def test_workspace_size_at_device_arithmetic_limits(L):
    """Shapes whose 32-bit device quantities would overflow are rejected
    (size 0), and the largest accepted ones still get a size."""
    # One cache block of 1024 x 8191 heads x 128 x 2 bytes fits 31 bits; 8192 heads do not.
    assert L.pa_attention_workspace_size(1, 8, 1, 8191, 8191, 128, 1024) > 0
    assert L.pa_attention_workspace_size(1, 8, 1, 8192, 8192, 128, 1024) == 0
    # 65536 sequences x 256 splits x 64 KV heads = 2^30 decode items (and 2^30
    # partial rows): accepted; 65 KV heads: rejected.
    assert L.pa_attention_workspace_size(65536, 65536, 16384, 64, 64, 128, 16) > 0
    assert L.pa_attention_workspace_size(65536, 65536, 16384, 65, 65, 128, 16) == 0


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails before a launch
FAKE_OUT = ctypes.c_void_p(0x10000000)   # an output range apart from every FAKE input


def _attn(L, **kw):
    a = dict(q=FAKE, cu=FAKE, lens=FAKE, table=FAKE, kc=FAKE, vc=FAKE, out=FAKE_OUT, B=2, T=5, MB=2,
             NB=8, scale=0.125, cap=0.0, win=0, hq=4, hk=2, d=64, bs=16, dtype=0, ws=FAKE, wsb=0,
             st=None)
    a.update(kw)
    return L.pa_attention(a["q"], a["cu"], a["lens"], a["table"], a["kc"], a["vc"], a["out"],
                          a["B"], a["T"], a["MB"], a["NB"], a["scale"], a["cap"], a["win"],
                          a["hq"], a["hk"], a["d"], a["bs"], a["dtype"], a["ws"], a["wsb"],
                          a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(d=256), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(bs=8), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(bs=48), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(dtype=7), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(hk=3), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(hq=256, hk=1), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(scale=float("nan")), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(cap=-1.0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(cap=float("nan")), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(cap=float("inf")), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(cap=1e-40, scale=1e30), _lib.PA_ERR_INVALID_ARGUMENT),   # scale / cap overflows
    (dict(B=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(T=-1), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(q=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(table=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(ws=None, wsb=1 << 30), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(ws=ctypes.c_void_p(0x1010), wsb=1 << 30), _lib.PA_ERR_INVALID_ARGUMENT),  # unaligned
    (dict(wsb=16), _lib.PA_ERR_WORKSPACE_TOO_SMALL),
    (dict(NB=1 << 28, bs=16), _lib.PA_ERR_NOT_IMPLEMENTED),   # slots beyond int32
    (dict(MB=16385, bs=16), _lib.PA_ERR_NOT_IMPLEMENTED),     # context beyond 262144 tokens
    (dict(hq=8192, hk=8192, MB=1, bs=1024, d=128), _lib.PA_ERR_NOT_IMPLEMENTED),  # block > 2^31 B
    (dict(B=65536, MB=16384, hq=65, hk=65, d=128), _lib.PA_ERR_NOT_IMPLEMENTED),  # > 2^30 items
    (dict(q=ctypes.c_void_p(0x1008), wsb=1 << 30), _lib.PA_ERR_INVALID_ARGUMENT),  # q unaligned
    (dict(out=ctypes.c_void_p(0x1002), wsb=1 << 30), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(vc=ctypes.c_void_p(0x1004), wsb=1 << 30), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(out=ctypes.c_void_p(0x1000 + 4 * 64 * 2), wsb=1 << 30),
     _lib.PA_ERR_INVALID_ARGUMENT),   # out overlaps q (from q's second row)
])
def test_attention_rejects_on_host(L, kw, status):
    assert _attn(L, **kw) == status
    assert L.pa_last_error() != b""


def test_attention_empty_call_is_ok(L):
    assert _attn(L, T=0, q=None, out=None, ws=None) == _lib.PA_OK


def _scatter(L, **kw):
    a = dict(k=FAKE, v=FAKE, slots=FAKE, kc=FAKE, vc=FAKE, T=5, NB=8, hk=2, d=64, bs=16, dtype=0)
    a.update(kw)
    return L.pa_scatter_kv(a["k"], a["v"], a["slots"], a["kc"], a["vc"], a["T"], a["NB"],
                           a["hk"], a["d"], a["bs"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=60), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(dtype=3), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(T=-2), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(hk=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(slots=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(NB=1 << 30, bs=16), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(k=ctypes.c_void_p(0x1008)), _lib.PA_ERR_INVALID_ARGUMENT),   # unaligned K rows
    (dict(vc=ctypes.c_void_p(0x1002)), _lib.PA_ERR_INVALID_ARGUMENT),
])
def test_scatter_rejects_on_host(L, kw, status):
    assert _scatter(L, **kw) == status


def test_scatter_empty_call_is_ok(L):
    assert _scatter(L, T=0, k=None, v=None, slots=None) == _lib.PA_OK


def _scatter_paged(L, **kw):
    a = dict(k=FAKE, v=FAKE, cu=FAKE, lens=FAKE, table=FAKE, kc=FAKE, vc=FAKE, B=2, T=5, MB=2,
             NB=8, hk=2, d=64, bs=16, dtype=0)
    a.update(kw)
    return L.pa_scatter_kv_paged(a["k"], a["v"], a["cu"], a["lens"], a["table"], a["kc"], a["vc"],
                                 a["B"], a["T"], a["MB"], a["NB"], a["hk"], a["d"], a["bs"],
                                 a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=60), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(dtype=2), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(T=-1), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(B=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(MB=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(hk=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(cu=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(table=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(NB=1 << 30, bs=16), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(MB=1 << 28, bs=16), _lib.PA_ERR_NOT_IMPLEMENTED),
])
def test_scatter_paged_rejects_on_host(L, kw, status):
    assert _scatter_paged(L, **kw) == status
    assert L.pa_last_error() != b""


def test_scatter_paged_empty_call_is_ok(L):
    assert _scatter_paged(L, T=0, k=None, v=None) == _lib.PA_OK


def _rot(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cos=FAKE, sin=FAKE, maxpos=64, rdim=64, inter=0, cu=FAKE,
             lens=FAKE, table=FAKE, qo=FAKE, kc=FAKE, vc=FAKE, B=2, T=5, MB=2, NB=8, hq=4, hk=2,
             d=64, bs=16, dtype=0)
    a.update(kw)
    return L.pa_rotary_scatter_kv(a["q"], a["k"], a["v"], a["cos"], a["sin"], a["maxpos"],
                                  a["rdim"], a["inter"], a["cu"], a["lens"], a["table"], a["qo"],
                                  a["kc"], a["vc"], a["B"], a["T"], a["MB"], a["NB"], a["hq"],
                                  a["hk"], a["d"], a["bs"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(d=60), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(rdim=24), _lib.PA_ERR_NOT_IMPLEMENTED),        # not a multiple of 16
    (dict(NB=1 << 30, bs=16), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(T=-1), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(B=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(hq=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(k=None), _lib.PA_ERR_INVALID_ARGUMENT),         # key without value
    (dict(sin=None), _lib.PA_ERR_INVALID_ARGUMENT),       # cos without sin
    (dict(rdim=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(rdim=80), _lib.PA_ERR_INVALID_ARGUMENT),        # beyond head_size
    (dict(maxpos=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(q=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(kc=None), _lib.PA_ERR_INVALID_ARGUMENT),        # (q_out may be null: Q not written)
    (dict(table=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(qo=ctypes.c_void_p(0x1008)), _lib.PA_ERR_INVALID_ARGUMENT),   # unaligned
    (dict(cos=ctypes.c_void_p(0x1004)), _lib.PA_ERR_INVALID_ARGUMENT),  # unaligned
])
def test_rotary_scatter_rejects_on_host(L, kw, status):
    assert _rot(L, **kw) == status
    assert L.pa_last_error() != b""


def _attn_rope(L, **kw):
    a = dict(q=FAKE, stride=8 * 64, cos=FAKE, sin=FAKE, maxpos=64, rdim=64, inter=0, cu=FAKE,
             lens=FAKE, table=FAKE, kc=FAKE, vc=FAKE, out=FAKE_OUT, B=2, T=5, MB=2, NB=8,
             scale=0.125, cap=0.0, win=0, hq=4, hk=2, d=64, bs=16, dtype=0, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return L.pa_attention_rope(a["q"], a["stride"], a["cos"], a["sin"], a["maxpos"], a["rdim"],
                               a["inter"], a["cu"], a["lens"], a["table"], a["kc"], a["vc"],
                               a["out"], a["B"], a["T"], a["MB"], a["NB"], a["scale"], a["cap"],
                               a["win"], a["hq"], a["hk"], a["d"], a["bs"], a["dtype"], a["ws"],
                               a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(stride=4 * 64 - 8), _lib.PA_ERR_INVALID_ARGUMENT),   # below num_heads * head_size
    (dict(stride=4 * 64 + 4), _lib.PA_ERR_INVALID_ARGUMENT),   # rows not 16-byte aligned
    (dict(stride=1 << 60), _lib.PA_ERR_INVALID_ARGUMENT),      # q's rows beyond 2^60 elements
    (dict(sin=None), _lib.PA_ERR_INVALID_ARGUMENT),            # cos without sin
    (dict(rdim=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(rdim=80), _lib.PA_ERR_INVALID_ARGUMENT),             # beyond head_size
    (dict(rdim=24), _lib.PA_ERR_NOT_IMPLEMENTED),              # not a multiple of 16
    (dict(maxpos=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(cos=ctypes.c_void_p(0x1004)), _lib.PA_ERR_INVALID_ARGUMENT),   # unaligned table
    (dict(q=ctypes.c_void_p(0x1008)), _lib.PA_ERR_INVALID_ARGUMENT),     # unaligned q
    (dict(d=96, stride=8 * 96), _lib.PA_ERR_NOT_IMPLEMENTED),  # pa_attention's own limits
    (dict(wsb=16), _lib.PA_ERR_WORKSPACE_TOO_SMALL),
    (dict(cap=-1.0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(out=ctypes.c_void_p(0x1000 + 4 * 8 * 64 * 2)), _lib.PA_ERR_INVALID_ARGUMENT),  # in q's rows
])
def test_attention_rope_rejects_on_host(L, kw, status):
    assert _attn_rope(L, **kw) == status
    assert L.pa_last_error() != b""


def test_attention_rope_empty_call_is_ok(L):
    assert _attn_rope(L, T=0, q=None, out=None, ws=None) == _lib.PA_OK
    # no tables: rotary_dim and max_position are not looked at
    assert _attn_rope(L, T=0, cos=None, sin=None, rdim=0, maxpos=0) == _lib.PA_OK


def _rot8(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cos=FAKE, sin=FAKE, maxpos=64, rdim=64, inter=0, cu=FAKE,
             lens=FAKE, table=FAKE, ks=FAKE, vs=FAKE, qo=FAKE_OUT, kc=FAKE, vc=FAKE, B=2, T=5, MB=2,
             NB=8, hq=4, hk=2, d=64, bs=16, dtype=0)
    a.update(kw)
    return L.pa_rotary_scatter_kv_fp8(a["q"], a["k"], a["v"], a["cos"], a["sin"], a["maxpos"],
                                      a["rdim"], a["inter"], a["cu"], a["lens"], a["table"],
                                      a["ks"], a["vs"], a["qo"], a["kc"], a["vc"], a["B"], a["T"],
                                      a["MB"], a["NB"], a["hq"], a["hk"], a["d"], a["bs"],
                                      a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ks=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(vs=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(vs=ctypes.c_void_p(0x1004)), _lib.PA_ERR_INVALID_ARGUMENT),   # unaligned scales
    (dict(rdim=24), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(d=60), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(q=None), _lib.PA_ERR_INVALID_ARGUMENT),        # Q needed: q_out given
])
def test_rotary_scatter_fp8_rejects_on_host(L, kw, status):
    assert _rot8(L, **kw) == status
    assert L.pa_last_error() != b""


def test_rotary_scatter_fp8_empty_call_is_ok(L):
    assert _rot8(L, T=0, q=None, qo=None) == _lib.PA_OK


def test_rotary_scatter_empty_call_is_ok(L):
    assert _rot(L, T=0, q=None, qo=None) == _lib.PA_OK
    # no tables: rotary_dim and max_position are not looked at
    assert _rot(L, T=0, cos=None, sin=None, rdim=0, maxpos=0) == _lib.PA_OK


def test_seqlens_from_past_rejects_on_host(L):
    assert L.pa_seqlens_from_past(FAKE, FAKE, FAKE, 0, None) == _lib.PA_ERR_INVALID_ARGUMENT
    assert L.pa_seqlens_from_past(FAKE, None, FAKE, 3, None) == _lib.PA_ERR_INVALID_ARGUMENT
    assert L.pa_seqlens_from_past(FAKE, FAKE, None, 3, None) == _lib.PA_ERR_INVALID_ARGUMENT


# ---------------------------------------------------------------- fp8 caches

def _scatter8(L, **kw):
    a = dict(k=FAKE, v=FAKE, slots=FAKE, ks=FAKE, vs=FAKE, kc=FAKE, vc=FAKE, T=5, NB=8, hk=2,
             d=64, bs=16, dtype=0, st=None)
    a.update(kw)
    return L.pa_scatter_kv_fp8(a["k"], a["v"], a["slots"], a["ks"], a["vs"], a["kc"], a["vc"],
                               a["T"], a["NB"], a["hk"], a["d"], a["bs"], a["dtype"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(d=60), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(T=-1), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(hk=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(ks=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(vs=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(kc=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(NB=1 << 30, bs=16), _lib.PA_ERR_NOT_IMPLEMENTED),
])
def test_scatter_fp8_rejects_on_host(L, kw, status):
    assert _scatter8(L, **kw) == status
    assert L.pa_last_error() != b""


def test_scatter_fp8_empty_call_is_ok(L):
    assert _scatter8(L, T=0, k=None, v=None, ks=None, vs=None) == _lib.PA_OK


def _attn8(L, **kw):
    a = dict(q=FAKE, cu=FAKE, lens=FAKE, table=FAKE, kc=FAKE, vc=FAKE, ks=FAKE, vs=FAKE, out=FAKE_OUT,
             B=2, T=5, mq=4, MB=2, NB=8, scale=0.125, cap=0.0, win=0, hq=4, hk=2, d=64, bs=16,
             dtype=0, ws=FAKE, wsb=0, st=None)
    a.update(kw)
    return L.pa_attention_fp8(a["q"], a["cu"], a["lens"], a["table"], a["kc"], a["vc"], a["ks"],
                              a["vs"], a["out"], a["B"], a["T"], a["mq"], a["MB"], a["NB"],
                              a["scale"], a["cap"], a["win"], a["hq"], a["hk"], a["d"], a["bs"],
                              a["dtype"], a["ws"], a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(mq=9), _lib.PA_ERR_NOT_IMPLEMENTED),          # 9 * G 2 = 18 columns > 16
    (dict(hq=34, mq=1), _lib.PA_ERR_NOT_IMPLEMENTED),   # G 17
    (dict(mq=-1), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(ks=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(vs=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(dtype=2), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(d=96), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(bs=24), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(scale=float("nan")), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(cap=-0.5), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(), _lib.PA_ERR_WORKSPACE_TOO_SMALL),
    (dict(cap=30.0, win=128), _lib.PA_ERR_WORKSPACE_TOO_SMALL),   # options accepted
])
def test_attention_fp8_rejects_on_host(L, kw, status):
    assert _attn8(L, **kw) == status
    assert L.pa_last_error() != b""


def test_attention_fp8_empty_call_is_ok(L):
    assert _attn8(L, T=0, mq=0) == _lib.PA_OK


def _scatter_paged8(L, **kw):
    a = dict(k=FAKE, v=FAKE, cu=FAKE, lens=FAKE, table=FAKE, ks=FAKE, vs=FAKE, kc=FAKE, vc=FAKE,
             B=2, T=5, MB=2, NB=8, hk=2, d=64, bs=16, dtype=0)
    a.update(kw)
    return L.pa_scatter_kv_paged_fp8(a["k"], a["v"], a["cu"], a["lens"], a["table"], a["ks"],
                                     a["vs"], a["kc"], a["vc"], a["B"], a["T"], a["MB"], a["NB"],
                                     a["hk"], a["d"], a["bs"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=60), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(dtype=2), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(T=-1), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(B=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(MB=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(hk=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(cu=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(ks=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(vs=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(ks=ctypes.c_void_p(0x1004)), _lib.PA_ERR_INVALID_ARGUMENT),   # unaligned scales
    (dict(kc=ctypes.c_void_p(0x1008)), _lib.PA_ERR_INVALID_ARGUMENT),   # unaligned cache
    (dict(NB=1 << 30, bs=16), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(MB=1 << 28, bs=16), _lib.PA_ERR_NOT_IMPLEMENTED),
])
def test_scatter_paged_fp8_rejects_on_host(L, kw, status):
    assert _scatter_paged8(L, **kw) == status
    assert L.pa_last_error() != b""


def test_scatter_paged_fp8_empty_call_is_ok(L):
    assert _scatter_paged8(L, T=0, k=None, v=None, ks=None, vs=None) == _lib.PA_OK


def _attn_rope8(L, **kw):
    a = dict(q=FAKE, stride=8 * 64, cos=FAKE, sin=FAKE, maxpos=64, rdim=64, inter=0, cu=FAKE,
             lens=FAKE, table=FAKE, kc=FAKE, vc=FAKE, ks=FAKE, vs=FAKE, out=FAKE_OUT, B=2, T=5,
             mq=4, MB=2, NB=8, scale=0.125, cap=0.0, win=0, hq=4, hk=2, d=64, bs=16, dtype=0,
             ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return L.pa_attention_rope_fp8(a["q"], a["stride"], a["cos"], a["sin"], a["maxpos"],
                                   a["rdim"], a["inter"], a["cu"], a["lens"], a["table"], a["kc"],
                                   a["vc"], a["ks"], a["vs"], a["out"], a["B"], a["T"], a["mq"],
                                   a["MB"], a["NB"], a["scale"], a["cap"], a["win"], a["hq"],
                                   a["hk"], a["d"], a["bs"], a["dtype"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(mq=9), _lib.PA_ERR_NOT_IMPLEMENTED),          # 9 * G 2 = 18 columns > 16
    (dict(mq=-1), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(ks=None), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(vs=ctypes.c_void_p(0x1004)), _lib.PA_ERR_INVALID_ARGUMENT),   # unaligned scales
    (dict(stride=4 * 64 - 8), _lib.PA_ERR_INVALID_ARGUMENT),   # below num_heads * head_size
    (dict(stride=4 * 64 + 4), _lib.PA_ERR_INVALID_ARGUMENT),   # rows not 16-byte aligned
    (dict(sin=None), _lib.PA_ERR_INVALID_ARGUMENT),            # cos without sin
    (dict(rdim=80), _lib.PA_ERR_INVALID_ARGUMENT),             # beyond head_size
    (dict(rdim=24), _lib.PA_ERR_NOT_IMPLEMENTED),              # not a multiple of 16
    (dict(maxpos=0), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(d=96, stride=8 * 96), _lib.PA_ERR_NOT_IMPLEMENTED),  # pa_attention's own limits
    (dict(wsb=16), _lib.PA_ERR_WORKSPACE_TOO_SMALL),
    (dict(out=ctypes.c_void_p(0x1000 + 4 * 8 * 64 * 2)), _lib.PA_ERR_INVALID_ARGUMENT),  # in q's rows
])
def test_attention_rope_fp8_rejects_on_host(L, kw, status):
    assert _attn_rope8(L, **kw) == status
    assert L.pa_last_error() != b""


def test_attention_rope_fp8_empty_call_is_ok(L):
    assert _attn_rope8(L, T=0, q=None, out=None, ws=None, mq=0) == _lib.PA_OK
    assert _attn_rope8(L, T=0, cos=None, sin=None, rdim=0, maxpos=0, mq=0) == _lib.PA_OK


def test_profile_kind_selection(L):
    """Profiling state is host-only: selecting kinds, enabling and reading
    with nothing recorded need no GPU; unknown kind names are rejected."""
    import paged_kv_cache_pa_amd as pa
    pa.profile_select(["attention"])
    pa.profile_enable(True)
    pa.profile_enable(False)
    assert all(v == (0.0, 0) for v in pa.profile_read().values())
    pa.profile_select(None)
    assert L.pa_profile_select(0xFFFFFFFF) == 0
    with pytest.raises(ValueError):
        pa.profile_select(["attention", "softmax"])


def _noalloc(L, **kw):
    a = dict(q=FAKE, cu=FAKE, lens=FAKE, table=FAKE, kc=FAKE, vc=FAKE, out=FAKE_OUT, B=2, T=5, MB=2,
             NB=8, scale=0.125, cap=0.0, win=0, hq=4, hk=2, d=64, bs=16, dtype=0, st=None)
    a.update(kw)
    return L.pa_attention_noalloc(a["q"], a["cu"], a["lens"], a["table"], a["kc"], a["vc"],
                                  a["out"], a["B"], a["T"], a["MB"], a["NB"], a["scale"],
                                  a["cap"], a["win"], a["hq"], a["hk"], a["d"], a["bs"],
                                  a["dtype"], a["st"])


@pytest.mark.parametrize("kw,status", [
    # The large mixed batch's sizes need 520 MiB of workspace > the 256 MiB scratch.
    (dict(B=256, T=8432, MB=2048, NB=500224, hq=64, hk=8, d=128, bs=16, dtype=1),
     _lib.PA_ERR_WORKSPACE_TOO_SMALL),
    (dict(hk=3), _lib.PA_ERR_INVALID_ARGUMENT),
    (dict(d=96), _lib.PA_ERR_NOT_IMPLEMENTED),
    (dict(dtype=5), _lib.PA_ERR_NOT_IMPLEMENTED),
])
def test_attention_noalloc_rejects_on_host(L, kw, status):
    assert _noalloc(L, **kw) == status
    assert L.pa_last_error() != b""


def test_attention_noalloc_empty_call_is_ok(L):
    assert _noalloc(L, T=0, q=None, out=None) == _lib.PA_OK
