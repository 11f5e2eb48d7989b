"""CPU checks of the C ABI: the library loads, exports every function that
include/*.h declares, and rejects bad host-side arguments before any
device work. No call here passes validation, so nothing is launched."""
import ctypes
import os
import re

import pytest
import torch

import paged_kv_cache_209_amd as pa
from paged_kv_cache_209_amd import _lib

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))

# Fake, 16-byte aligned, never dereferenced pointers: every call below fails a
# host-side check before any launch.
P = 0x10000
INVALID, UNSUP, WS = pa.PA_ERR_INVALID_ARG, pa.PA_ERR_UNSUPPORTED, pa.PA_ERR_WORKSPACE


def _declared():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    lib = pa.library()
    names = _declared()
    assert len(names) >= 22
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"binding lacks {n}"


def test_version_and_status_strings():
    assert pa.version().startswith("pagedattn")
    lib = pa.library()
    for s in (0, -1, -2, -3, -4, -5):
        assert lib.pa_status_string(s)
    assert b"unknown" in lib.pa_status_string(7)


def kv(**kw):
    a = dict(kc=P, vc=P, k=P, v=P, slots=P, T=4, hkv=2, d=128, bs=256, nb=8, dt=pa.PA_BF16)
    a.update(kw)
    return pa.library().pa_kv_store(a["kc"], a["vc"], a["k"], a["v"], a["slots"], a["T"], a["hkv"], a["d"], a["bs"],
                                     a["nb"], a["dt"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(kc=None), INVALID), (dict(v=None), INVALID), (dict(slots=None), INVALID),
    (dict(T=-1), INVALID), (dict(hkv=0), INVALID), (dict(nb=0), INVALID), (dict(dt=5), INVALID),
    (dict(d=96), UNSUP), (dict(bs=128), UNSUP), (dict(nb=1 << 23), INVALID), (dict(k=P + 8), INVALID),
])
def test_kv_store_validation(kw, expect):
    assert kv(**kw) == expect


def test_kv_store_empty_is_noop():
    # zero tokens: nothing to launch, k/v/slots may be null
    assert kv(T=0, k=None, v=None, slots=None) == pa.PA_OK


def rope(**kw):
    a = dict(qo=P, kc=P, vc=P, q=P, k=P, v=P, pos=P, slots=P, T=4, hq=8, hkv=2, d=128, bs=256, nb=8, theta=1.0e6,
             dt=pa.PA_BF16)
    a.update(kw)
    return pa.library().pa_rope_kv_store(a["qo"], a["kc"], a["vc"], a["q"], a["k"], a["v"], a["pos"], a["slots"],
                                         a["T"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["theta"], a["dt"],
                                         None)


@pytest.mark.parametrize("kw,expect", [
    (dict(qo=None), INVALID), (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(pos=None), INVALID), (dict(slots=None), INVALID), (dict(kc=None), INVALID), (dict(T=-1), INVALID),
    (dict(hq=0), INVALID), (dict(hq=6, hkv=4), INVALID), (dict(theta=0.0), INVALID), (dict(theta=-2.0), INVALID),
    (dict(theta=float("nan")), INVALID), (dict(theta=float("inf")), INVALID), (dict(d=96), UNSUP),
    (dict(bs=64), UNSUP), (dict(dt=9), INVALID), (dict(qo=P + 4), INVALID), (dict(k=P + 8), INVALID),
])
def test_rope_kv_store_validation(kw, expect):
    assert rope(**kw) == expect


def test_rope_kv_store_empty_is_noop():
    assert rope(T=0, qo=None, q=None, k=None, v=None, pos=None, slots=None) == pa.PA_OK


def dec(**kw):
    a = dict(out=P, q=P, kc=P, vc=P, bt=P, cl=P, B=4, hq=8, hkv=2, d=128, bs=256, nb=64, mb=16, mc=4096,
             scale=0.088, dt=pa.PA_BF16, part=0, ws=None, wsb=0)
    a.update(kw)
    return pa.library().pa_paged_attn_decode_ex(
        a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["B"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"],
        a["mb"], a["mc"], a["scale"], a["dt"], a["part"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(bt=None), INVALID), (dict(cl=None), INVALID), (dict(kc=None), INVALID),
    (dict(hq=6, hkv=4), INVALID), (dict(hq=0), INVALID), (dict(B=-1), INVALID), (dict(mc=0), INVALID),
    (dict(mc=4097), INVALID), (dict(mb=0), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID), (dict(part=-1), INVALID), (dict(part=-256), INVALID),
    (dict(d=80), UNSUP), (dict(bs=16), UNSUP), (dict(dt=3), INVALID), (dict(out=P + 4), INVALID),
    (dict(ws=None, wsb=0), WS), (dict(ws=P, wsb=1024), WS),
])
def test_decode_validation(kw, expect):
    assert dec(**kw) == expect


def test_decode_empty_batch_is_noop():
    assert dec(B=0, out=None, q=None, bt=None, cl=None) == pa.PA_OK


def test_decode_workspace_sizing():
    # one 64-token work unit per context: nothing is ever split
    assert pa.decode_workspace_bytes(4, 8, 128, 64) == 0
    need = pa.decode_workspace_bytes(4, 8, 128, 65)
    # counters (padded) + two piece slots per workgroup of the largest grid
    # (2048), each for up to 4 query heads: lse values and partial outputs
    assert need >= 2 * 2048 * 4 * (128 + 1) * 4
    # independent of the context length
    assert pa.decode_workspace_bytes(4, 8, 128, 1 << 20) == need
    assert dec(ws=P, wsb=need - 1) == WS
    assert dec(ws=P, wsb=need - 1, part=7) == WS
    assert dec(ws=P, wsb=need, part=2049) == INVALID
    n = pa.decode_num_workgroups(64, 16, 8, 128, 4096)
    assert 1 <= n <= 64 * 8 * 16
    assert pa.decode_num_workgroups(1, 2, 1, 64, 1, torch.float32) == 1
    assert pa.decode_num_workgroups(1, 2, 1, 96, 100) == 0
    # small batches: at most 8 workgroups per (sequence, query-head group) item
    assert pa.decode_num_workgroups(1, 16, 8, 128, 4096) <= 8 * 8
    assert pa.decode_num_workgroups(2, 32, 8, 128, 8192) <= 2 * 8 * 8


def pre(**kw):
    a = dict(out=P, q=P, k=P, v=P, kc=P, vc=P, bt=P, cl=P, cu=P, B=2, tq=10, mq=5, hq=8, hkv=2, d=128, bs=256,
             nb=64, mb=16, mc=4096, scale=0.088, dt=pa.PA_BF16, ws=None, wsb=0)
    a.update(kw)
    return pa.library().pa_paged_attn_prefill(
        a["out"], a["q"], a["k"], a["v"], a["kc"], a["vc"], a["bt"], a["cl"], a["cu"], a["B"], a["tq"], a["mq"],
        a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["mb"], a["mc"], a["scale"], a["dt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(dt=pa.PA_F32), UNSUP), (dict(d=96), UNSUP), (dict(bs=64), UNSUP), (dict(dt=9), INVALID),
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(cu=None), INVALID), (dict(vc=None), INVALID),
    (dict(hq=6, hkv=4), INVALID), (dict(mq=5000), INVALID), (dict(mc=4097), INVALID), (dict(B=-1), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(v=P + 2), INVALID),
    (dict(ws=None), WS), (dict(ws=P, wsb=4096), WS),
])
def test_prefill_validation(kw, expect):
    assert pre(**kw) == expect


def pre_ex(grid, **kw):
    a = dict(out=P, q=P, k=P, v=P, kc=P, vc=P, bt=P, cl=P, cu=P, B=2, tq=10, mq=5, hq=8, hkv=2, d=128, bs=256,
             nb=64, mb=16, mc=4096, scale=0.088, dt=pa.PA_BF16, ws=None, wsb=0)
    a.update(kw)
    return pa.library().pa_paged_attn_prefill_ex(
        a["out"], a["q"], a["k"], a["v"], a["kc"], a["vc"], a["bt"], a["cl"], a["cu"], a["B"], a["tq"], a["mq"],
        a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["mb"], a["mc"], a["scale"], a["dt"], grid, a["ws"], a["wsb"],
        None)


def test_prefill_ex_grid_argument():
    """A negative grid is rejected before anything else; 0 and positive grids
    pass to the same checks as pa_paged_attn_prefill (here: no workspace)."""
    assert pre_ex(-1) == INVALID
    assert pre_ex(-1, B=0) == INVALID
    assert pre_ex(0) == WS and pre_ex(7) == WS and pre_ex(100000) == WS
    assert pre_ex(3, B=0) == pa.PA_OK
    assert pre_ex(3, dt=pa.PA_F32) == UNSUP


def test_prefill_empty_is_noop_and_workspace_sizing():
    assert pre(tq=0, out=None, q=None, k=None, v=None) == pa.PA_OK
    assert pre(B=0) == pa.PA_OK
    need = pa.prefill_workspace_bytes(2, 8, 128, 5, 4096)
    assert need > 0
    assert pre(ws=P, wsb=need - 16) == WS


def test_decode_graphs_validation():
    """Argument checks of pa_decode_graphs_create run before any HIP call."""
    import ctypes

    from paged_kv_cache_209_amd.decode_graphs import _Buffers

    lib = pa.library()
    h = ctypes.c_void_p()

    def create(bufs, max_batch=4, hq=8, hkv=2, d=128, bs=256, nb=8, mb=4, dt=pa.PA_BF16, out=True):
        return lib.pa_decode_graphs_create(None if bufs is None else ctypes.addressof(bufs), max_batch, hq, hkv, d,
                                           bs, nb, mb, 0.1, dt, ctypes.addressof(h) if out else None)

    good = _Buffers(P, P, P, P, P, P, P, P, P, P, 1 << 30)
    assert create(good, out=False) == INVALID
    assert create(None) == INVALID
    assert create(good, max_batch=0) == INVALID
    assert create(good, max_batch=513) == INVALID
    assert create(good, d=96) == UNSUP
    assert create(good, bs=128) == UNSUP
    assert create(good, hq=6, hkv=4) == INVALID
    assert create(_Buffers(P, P, P, P, None, P, P, P, P, P, 1 << 30)) == INVALID
    assert create(_Buffers(P, P, P, P, P, P, P, P, P, None, 0)) == WS
    assert create(_Buffers(P, P, P, P, P, P, P, P, P, P, 1024)) == WS
    assert lib.pa_decode_graphs_launch(None, 1, None) == INVALID
    assert lib.pa_decode_graphs_bucket(None, 1) == 0
    lib.pa_decode_graphs_destroy(None)


def test_fp8_validation():
    lib = pa.library()

    def store(**kw):
        a = dict(kc=P, vc=P, k=P, v=P, slots=P, T=4, hkv=2, d=128, bs=256, nb=8, ks=0.1, vs=0.1)
        a.update(kw)
        return lib.pa_kv_store_fp8(a["kc"], a["vc"], a["k"], a["v"], a["slots"], a["T"], a["hkv"], a["d"], a["bs"],
                                   a["nb"], a["ks"], a["vs"], None)

    assert store(kc=None) == INVALID
    assert store(d=64) == UNSUP
    assert store(ks=0.0) == INVALID and store(vs=-1.0) == INVALID and store(ks=float("inf")) == INVALID
    assert store(T=0, k=None) == pa.PA_OK
    assert store(k=P + 4) == INVALID

    def dec(**kw):
        a = dict(out=P, q=P, kc=P, vc=P, bt=P, cl=P, B=2, hq=8, hkv=2, d=128, bs=256, nb=8, mb=4, mc=1000,
                 scale=0.1, ks=0.1, vs=0.1, ws=P, wsb=1 << 30)
        a.update(kw)
        return lib.pa_paged_attn_decode_fp8(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["B"], a["hq"],
                                            a["hkv"], a["d"], a["bs"], a["nb"], a["mb"], a["mc"], a["scale"], a["ks"],
                                            a["vs"], a["ws"], a["wsb"], None)

    assert dec(d=64) == UNSUP
    assert dec(hq=6, hkv=4) == INVALID
    assert dec(mc=4 * 256 + 1) == INVALID
    assert dec(ks=0.0) == INVALID
    assert dec(ws=None) == WS
    assert dec(wsb=16) == WS
    assert dec(B=0, out=None) == pa.PA_OK
    need = pa.decode_fp8_workspace_bytes(2, 8, 128, 1000)
    assert need == pa.decode_fp8_workspace_bytes(2, 8, 128, 1024) > 0
    assert pa.decode_fp8_workspace_bytes(2, 8, 64, 1000) == 0
    # the fp8 decode shares the decode kernel and its workspace rule
    assert need == pa.decode_workspace_bytes(2, 8, 128, 1000)


def test_qknorm_rope_validation():
    lib = pa.library()

    def call(**kw):
        a = dict(qo=P, kc=P, vc=P, q=P, k=P, v=P, qw=P, kw=P, eps=1e-6, pos=P, slots=P, T=4, hq=4, hkv=2, d=128,
                 bs=256, nb=8, theta=1e6, dt=pa.PA_BF16)
        a.update(kw)
        return lib.pa_qknorm_rope_kv_store(a["qo"], a["kc"], a["vc"], a["q"], a["k"], a["v"], a["qw"], a["kw"],
                                           a["eps"], a["pos"], a["slots"], a["T"], a["hq"], a["hkv"], a["d"], a["bs"],
                                           a["nb"], a["theta"], a["dt"], None)

    assert call(qw=None) == INVALID and call(kw=None) == INVALID
    assert call(qw=P + 8) == INVALID
    assert call(eps=-1.0) == INVALID and call(eps=float("nan")) == INVALID
    assert call(d=96) == UNSUP
    assert call(theta=0.0) == INVALID
    assert call(T=0, q=None) == pa.PA_OK


def fused(**kw):
    a = dict(out=P, q=P, kc=P, vc=P, kn=P, vn=P, sl=P, bt=P, cl=P, B=4, hq=8, hkv=2, d=128, bs=256, nb=64, mb=16,
             mc=4096, scale=0.088, dt=pa.PA_BF16, ws=None, wsb=0)
    a.update(kw)
    return pa.library().pa_paged_attn_decode_store(
        a["out"], a["q"], a["kc"], a["vc"], a["kn"], a["vn"], a["sl"], a["bt"], a["cl"], a["B"], a["hq"], a["hkv"],
        a["d"], a["bs"], a["nb"], a["mb"], a["mc"], a["scale"], a["dt"], a["ws"], a["wsb"], None)


def test_decode_store_validation():
    """The one-launch decode step rejects what pa_paged_attn_decode rejects,
    plus missing or misaligned new-token rows and slot_mapping; an empty batch
    is a no-op."""
    for kw in (dict(kn=None), dict(vn=None), dict(sl=None), dict(kn=P + 8), dict(vn=P + 2), dict(q=None),
               dict(bt=None), dict(hq=6, hkv=4), dict(mc=0), dict(scale=float("nan")), dict(dt=3)):
        assert fused(**kw) == INVALID, kw
    assert fused(d=80) == UNSUP
    assert fused(ws=None, wsb=0) == WS
    assert fused(B=0, out=None, q=None, kn=None, vn=None, sl=None, bt=None, cl=None) == pa.PA_OK


def test_workspace_status_validation():
    """pa_workspace_status rejects a missing or headerless workspace before
    any HIP call (it is a diagnostic that synchronises the stream)."""
    lib = pa.library()
    assert lib.pa_workspace_status(None, 1 << 20, None) == INVALID
    assert lib.pa_workspace_status(P, 255, None) == INVALID
    pa.check_workspace(None)  # no workspace: nothing to check


def test_workspace_layout_has_header_and_wide_counters():
    """Decode: 256-byte header, partial regions for the largest grid, then
    8 bytes per (sequence, query head); prefill likewise per counter."""
    a = pa.decode_workspace_bytes(4, 8, 128, 65)
    b = pa.decode_workspace_bytes(5, 8, 128, 65)
    assert b - a == 8 * 8
    assert a >= 256 + 2 * 2048 * 4 * (128 + 1) * 4 + 4 * 8 * 8
    p1 = pa.prefill_workspace_bytes(2, 8, 128, 5, 4096)
    p2 = pa.prefill_workspace_bytes(3, 8, 128, 5, 4096)
    assert p2 - p1 == 8 * 8 * 6


def _cpu(shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _decode_args(**kw):
    a = dict(out=_cpu((4, 8, 128)), q=_cpu((4, 8, 128)), kc=_cpu((3, 256, 2, 128)), vc=_cpu((3, 256, 2, 128)),
             bt=_cpu((4, 2), torch.int32), cl=_cpu((4,), torch.int32))
    a.update(kw)
    return a


@pytest.mark.parametrize("kw", [
    dict(out=_cpu((4, 8, 64))), dict(out=_cpu((3, 8, 128))), dict(q=_cpu((4, 8, 64)), out=_cpu((4, 8, 64))),
    dict(vc=_cpu((4, 256, 2, 128))), dict(bt=_cpu((3, 2), torch.int32)), dict(bt=_cpu((4,), torch.int32)),
    dict(cl=_cpu((5,), torch.int32)), dict(q=_cpu((4, 1024))),
], ids=["out_d", "out_b", "q_d_vs_pool", "pools_differ", "bt_rows", "bt_1d", "cl_len", "q_2d"])
def test_decode_binding_rejects_mismatched_shapes(kw):
    a = _decode_args(**kw)
    with pytest.raises(ValueError, match="paged_attn_decode"):
        pa.paged_attn_decode(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], 0.1, 512)


def test_decode_binding_shapes_pass_then_device_check():
    a = _decode_args()
    with pytest.raises(ValueError, match="GPU tensor"):
        pa.paged_attn_decode(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], 0.1, 512)


def _prefill_args(**kw):
    a = dict(out=_cpu((10, 8, 128)), q=_cpu((10, 8, 128)), k=_cpu((10, 2, 128)), v=_cpu((10, 2, 128)),
             kc=_cpu((3, 256, 2, 128)), vc=_cpu((3, 256, 2, 128)), bt=_cpu((2, 2), torch.int32),
             cl=_cpu((2,), torch.int32), cu=_cpu((3,), torch.int32))
    a.update(kw)
    return a


@pytest.mark.parametrize("kw", [
    dict(out=_cpu((9, 8, 128))), dict(k=_cpu((10, 4, 128))), dict(v=_cpu((9, 2, 128))),
    dict(q=_cpu((10, 8, 64)), out=_cpu((10, 8, 64))), dict(vc=_cpu((3, 256, 1, 128))),
    dict(bt=_cpu((3, 2), torch.int32)), dict(cu=_cpu((2,), torch.int32)), dict(cl=_cpu((2, 1), torch.int32)),
], ids=["out_rows", "k_heads", "v_rows", "q_d_vs_pool", "pools_differ", "bt_rows", "cu_len", "cl_2d"])
def test_prefill_binding_rejects_mismatched_shapes(kw):
    a = _prefill_args(**kw)
    with pytest.raises(ValueError, match="paged_attn_prefill"):
        pa.paged_attn_prefill(a["out"], a["q"], a["k"], a["v"], a["kc"], a["vc"], a["bt"], a["cl"], a["cu"], 0.1,
                              5, 512)


def test_prefill_binding_shapes_pass_then_device_check():
    a = _prefill_args()
    with pytest.raises(ValueError, match="GPU tensor"):
        pa.paged_attn_prefill(a["out"], a["q"], a["k"], a["v"], a["kc"], a["vc"], a["bt"], a["cl"], a["cu"], 0.1,
                              5, 512)
