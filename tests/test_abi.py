"""The C ABI without a GPU: exports, error strings, host-side argument checks.

Every call here fails validation (or has T = 0) and returns before anything
is launched, so no HIP device is needed.  Fake non-NULL pointers are never
dereferenced on those paths.
"""
import ctypes
import os
import re

import pytest

import quantized_moe_expert_amd as m
from quantized_moe_expert_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_q4.h")
FAKE = 0x10000  # never dereferenced


def header_functions():
    text = open(HEADER).read()
    return re.findall(r"MOE_Q4_API\s+[\w\s\*]+?\b(moe_q4_\w+)\s*\(", text)


def test_every_declared_function_is_exported():
    names = header_functions()
    assert len(names) == 23
    assert set(names) == set(m.EXPORTS)
    lib = m.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_error_strings():
    assert m.error_string(0) == "ok"
    for st in (-1, -2, -3, -4):
        assert m.error_string(st) not in ("ok", "unknown status")
    assert m.error_string(7) == "unknown status"


def test_workspace_sizes():
    assert m.workspace_size(m.WS_ROUTE, 16, 256, 8, 2048, 512) == 0
    assert m.workspace_size(m.WS_DECODE, 0, 256, 8, 2048, 512) == 0
    d1 = m.workspace_size(m.WS_DECODE, 1, 256, 8, 2048, 512)
    d16 = m.workspace_size(m.WS_DECODE, 16, 256, 8, 2048, 512)
    assert 0 < d1 < d16
    # decode keeps the grouping (counts, offsets, permutation, tiles) only
    assert d16 >= 16 * 8 * 4 * 2
    p = m.workspace_size(m.WS_PREFILL, 4096, 256, 8, 2048, 512)
    assert p >= 4096 * 8 * 512 * 2          # f16 h
    assert m.workspace_size(m.WS_GROUP, 4096, 256, 8, 64, 64) >= 4096 * 8 * 4 * 2


def _layer(fmt=0, E=256, H=2048, I=512, null=None):
    ptrs = {n: FAKE for n in ("gate_q", "up_q", "down_q", "gate_sm", "up_sm", "down_sm")}
    if null:
        ptrs[null] = None
    return _lib.Layer(E, H, I, fmt, *[ptrs[n] for n in ("gate_q", "up_q", "down_q", "gate_sm", "up_sm", "down_sm")])


def _decode(layer, T=4, k=8, ws_bytes=1 << 30, x=FAKE, prefill=False):
    fn = m.lib().moe_q4_prefill if prefill else m.lib().moe_q4_decode
    return fn(x, FAKE, FAKE, T, k, ctypes.byref(layer), FAKE, FAKE, ws_bytes, None)


def test_route_validation():
    L = m.lib()
    r = lambda **kw: L.moe_q4_route(kw.get("x", FAKE), kw.get("w", FAKE), None, kw.get("lg", FAKE),
                                    kw.get("T", 4), kw.get("H", 2048), kw.get("E", 256), kw.get("k", 8),
                                    kw.get("idx", FAKE), kw.get("gate", FAKE), None, 0, None)
    assert r(lg=None) == _lib.ERR_INVALID_ARG
    assert r(idx=None) == _lib.ERR_INVALID_ARG
    assert r(w=None) == _lib.ERR_INVALID_ARG            # x given without router weights
    assert r(k=0) == _lib.ERR_INVALID_ARG
    assert r(k=9, E=8) == _lib.ERR_INVALID_ARG
    assert r(T=-1) == _lib.ERR_INVALID_ARG
    assert r(E=2048, k=8) == _lib.ERR_UNSUPPORTED
    assert r(k=33, E=256) == _lib.ERR_UNSUPPORTED
    assert r(H=4096) == _lib.ERR_UNSUPPORTED
    assert r(H=100) == _lib.ERR_UNSUPPORTED
    assert r(T=0) == _lib.OK


def test_group_validation():
    L = m.lib()
    g = lambda T=16, k=8, E=256, ws=FAKE, nb=1 << 30, cnt=FAKE: L.moe_q4_group(FAKE, T, k, E, cnt, FAKE, FAKE,
                                                                                  FAKE, ws, nb, None)
    assert g(cnt=None) == _lib.ERR_INVALID_ARG
    assert g(ws=None) == _lib.ERR_WORKSPACE
    assert g(nb=16) == _lib.ERR_WORKSPACE
    assert g(T=0) == _lib.OK
    assert g(k=300, E=256) == _lib.ERR_INVALID_ARG


def test_layer_validation():
    assert _decode(_layer(null="down_sm")) == _lib.ERR_INVALID_ARG
    assert _decode(_layer(fmt=4)) == _lib.ERR_UNSUPPORTED       # unknown format
    assert _decode(_layer(H=3072)) == _lib.ERR_UNSUPPORTED       # not a power of two
    assert _decode(_layer(H=4096)) == _lib.ERR_UNSUPPORTED       # above 2048
    assert _decode(_layer(fmt=1, I=64)) == _lib.ERR_UNSUPPORTED  # not a multiple of 128
    assert _decode(_layer(E=0)) == _lib.ERR_INVALID_ARG
    assert _decode(_layer(), x=None) == _lib.ERR_INVALID_ARG
    assert _decode(_layer(), ws_bytes=100) == _lib.ERR_WORKSPACE
    assert _decode(_layer(), k=0) == _lib.ERR_INVALID_ARG
    assert _decode(_layer(), T=0) == _lib.OK
    assert _decode(_layer(I=64), prefill=True) == _lib.ERR_UNSUPPORTED    # prefill needs I % 128 == 0
    assert _decode(_layer(H=128, I=128), prefill=True) == _lib.ERR_UNSUPPORTED  # and H % 256 == 0
    assert _decode(_layer(), prefill=True, ws_bytes=100) == _lib.ERR_WORKSPACE
    assert _decode(_layer(), prefill=True, T=0) == _lib.OK
    # pointer alignment: codes and activations 16 bytes, scale arrays 4 bytes
    lay = _layer()
    lay.up_q = FAKE + 8
    assert _decode(lay) == _lib.ERR_INVALID_ARG
    lay = _layer()
    lay.down_sm = FAKE + 2
    assert _decode(lay, prefill=True) == _lib.ERR_INVALID_ARG
    assert _decode(_layer(), x=FAKE + 4) == _lib.ERR_INVALID_ARG
    # prefill offsets are 32-bit: T * H, T * k * I and T * k * H below 2^31
    assert _decode(_layer(), prefill=True, T=1 << 20) == _lib.ERR_UNSUPPORTED
    assert _decode(_layer(H=256, I=2048), prefill=True, T=1 << 17, k=8) == _lib.ERR_UNSUPPORTED
    assert _decode(_layer(H=2048, I=256), prefill=True, T=1 << 17, k=8) == _lib.ERR_UNSUPPORTED
    # timed variants: events are required and must be non-NULL
    L = m.lib()
    ev_null = (ctypes.c_void_p * 4)(FAKE, FAKE, None, FAKE)
    ev_ok = (ctypes.c_void_p * 4)(*([FAKE] * 4))
    lay = _layer()
    for fn in (L.moe_q4_decode_timed, L.moe_q4_prefill_timed):
        assert fn(FAKE, FAKE, FAKE, 4, 8, ctypes.byref(lay), FAKE, FAKE, 1 << 30, None, None) == _lib.ERR_INVALID_ARG
        assert fn(FAKE, FAKE, FAKE, 4, 8, ctypes.byref(lay), FAKE, FAKE, 1 << 30, None, ev_null) == _lib.ERR_INVALID_ARG
        assert fn(FAKE, FAKE, FAKE, 4, 8, ctypes.byref(lay), FAKE, FAKE, 100, None, ev_ok) == _lib.ERR_WORKSPACE
        assert fn(FAKE, FAKE, FAKE, 0, 8, ctypes.byref(lay), FAKE, FAKE, 1 << 30, None, ev_ok) == _lib.OK


def test_forward_validation():
    L = m.lib()
    lay = _layer()
    f = lambda x=FAKE, ry=None, xo=None, lg=FAKE, T=4, k=8, ws=FAKE, nb=1 << 30, layer=lay: L.moe_q4_forward(
        x, ry, xo, FAKE, None, lg, T, k, ctypes.byref(layer), FAKE, FAKE, FAKE, ws, nb, None)
    assert f(x=None) == _lib.ERR_INVALID_ARG
    assert f(lg=None) == _lib.ERR_INVALID_ARG
    assert f(ry=FAKE, xo=None) == _lib.ERR_INVALID_ARG   # residual needs x_out
    assert f(ws=None) == _lib.ERR_WORKSPACE
    assert f(nb=64) == _lib.ERR_WORKSPACE
    assert f(T=0) == _lib.OK
    assert f(layer=_layer(fmt=4)) == _lib.ERR_UNSUPPORTED
    assert f(T=500, layer=_layer(I=64)) == _lib.ERR_UNSUPPORTED  # prefill path shape rules
    assert f(T=1 << 20) == _lib.ERR_UNSUPPORTED                  # prefill path 32-bit offsets
    assert f(x=FAKE + 2) == _lib.ERR_INVALID_ARG                 # misaligned activations
    assert f(ry=FAKE, xo=FAKE + 8) == _lib.ERR_INVALID_ARG
    assert m.workspace_size(m.WS_FORWARD, 16, 256, 8, 2048, 512) >= 2048
    ev_null = (ctypes.c_void_p * 4)(FAKE, None, FAKE, FAKE)
    ft = lambda ev, T=4: L.moe_q4_forward_timed(FAKE, None, None, FAKE, None, FAKE, T, 8, ctypes.byref(lay), FAKE,
                                                FAKE, FAKE, FAKE, 1 << 30, None, ev)
    assert ft(None) == _lib.ERR_INVALID_ARG     # events required
    assert ft(ev_null) == _lib.ERR_INVALID_ARG  # and non-NULL
    assert ft((ctypes.c_void_p * 4)(*([FAKE] * 4)), T=0) == _lib.OK
    assert L.moe_q4_workspace_init(None, 0, None) == _lib.ERR_WORKSPACE
    # the entry point on the library's own workspace: the same checks, and
    # shapes whose forward workspace exceeds its fixed size are refused before
    # any device call
    fn = lambda x=FAKE, ry=None, xo=None, T=4, k=8, layer=lay: L.moe_q4_forward_noalloc(
        x, ry, xo, FAKE, None, FAKE, T, k, ctypes.byref(layer), FAKE, FAKE, FAKE, None)
    assert fn(T=0) == _lib.OK
    assert fn(x=None) == _lib.ERR_INVALID_ARG
    assert fn(ry=FAKE, xo=None) == _lib.ERR_INVALID_ARG
    assert fn(layer=_layer(fmt=4)) == _lib.ERR_UNSUPPORTED
    big = m.workspace_size(m.WS_FORWARD, 4096, 256, 8, 2048, 512)
    assert big > m.NOALLOC_SCRATCH_BYTES
    assert fn(T=4096) == _lib.ERR_WORKSPACE
    # every decode-path shape fits: 64 tokens x top-16 (1024 pairs) at H = I = 2048, E = 1024
    assert m.workspace_size(m.WS_FORWARD, 64, 1024, 16, 2048, 2048) <= m.NOALLOC_SCRATCH_BYTES
    assert L.moe_q4_workspace_init(FAKE, 100, None) == _lib.ERR_WORKSPACE


def test_frame_validation():
    """moe_q4_frame checks every layer and lane before its first launch."""
    L = m.lib()
    P = ctypes.c_void_p

    def call(T=16, n=2, lanes=2, layers=None, routers=None, x=FAKE, xc=FAKE, nb=1 << 30, ws=FAKE, streams=None,
             events=None):
        layers = layers or [_layer() for _ in range(n)]
        lay = (_lib.Layer * len(layers))(*layers)
        rw = (P * n)(*(routers or [FAKE] * n))
        sts = (P * max(lanes, 1))(*([None] * max(lanes, 1))) if streams is None else streams
        return L.moe_q4_frame(x, T, 8, n, lay, rw, None, xc, FAKE, FAKE, FAKE, FAKE, lanes, sts, ws, nb, events)

    assert call(T=0) == _lib.OK
    assert call(n=0, layers=[_layer()]) == _lib.ERR_INVALID_ARG
    assert call(lanes=0) == _lib.ERR_INVALID_ARG
    assert call(lanes=m.FRAME_MAX_LANES + 1) == _lib.ERR_INVALID_ARG
    assert call(T=1, lanes=2) == _lib.ERR_INVALID_ARG           # more lanes than tokens
    assert call(x=None) == _lib.ERR_INVALID_ARG
    assert call(xc=None) == _lib.ERR_INVALID_ARG                # two layers need the chain
    assert call(routers=[FAKE, None]) == _lib.ERR_INVALID_ARG
    assert call(layers=[_layer(), _layer(I=256)]) == _lib.ERR_INVALID_ARG  # one shape per frame
    assert call(layers=[_layer(), _layer(fmt=4)]) == _lib.ERR_UNSUPPORTED  # layer 1 checked before any launch
    assert call(layers=[_layer(), _layer(null="down_q")]) == _lib.ERR_INVALID_ARG
    assert call(ws=None) == _lib.ERR_WORKSPACE
    need = m.frame_workspace_size(16, 256, 8, 2048, 512, 0, 2)
    assert need >= 2 * m.workspace_size(m.WS_FORWARD, 8, 256, 8, 2048, 512)
    assert call(nb=need - 1) == _lib.ERR_WORKSPACE
    assert call(x=FAKE + 2) == _lib.ERR_INVALID_ARG             # misaligned activations
    assert L.moe_q4_frame(FAKE, 16, 8, 2, None, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, 2, None, FAKE, 1 << 30,
                          None) == _lib.ERR_INVALID_ARG
    ev = (P * (2 * 2 * m.STAGE_EVENTS))(*([FAKE] * 15 + [None]))
    assert call(events=ev) == _lib.ERR_INVALID_ARG
    # sizes: lanes split the tokens as evenly as possible; out-of-range asks give 0
    assert m.frame_workspace_size(5, 256, 8, 2048, 512, 0, 2) == 2 * m.frame_workspace_size(3, 256, 8, 2048, 512,
                                                                                             0, 1)
    assert m.frame_workspace_size(16, 256, 8, 2048, 512, 0, 0) == 0
    assert m.frame_workspace_size(2, 256, 8, 2048, 512, 0, 3) == 0
    assert m.frame_workspace_size(16, 256, 8, 2048, 512, 512, 1) > m.frame_workspace_size(16, 256, 8, 2048, 512, 0,
                                                                                          1)


def test_forward_det_validation():
    """The slot-ordered decode entry point: its workspace adds the [T*k][H] fp32 routed rows on the decode
    path only, and it refuses a workspace sized for moe_q4_forward."""
    L = m.lib()
    lay = _layer()
    for T, k in ((1, 8), (16, 8), (64, 16)):
        base = m.workspace_size(m.WS_FORWARD, T, 256, k, 2048, 512)
        det = m.workspace_size(m.WS_FORWARD_DET, T, 256, k, 2048, 512)
        assert det >= base + T * k * 2048 * 4
        assert det <= base + T * k * 2048 * 4 + 4096
    assert m.workspace_size(m.WS_FORWARD_DET, 4096, 256, 8, 2048, 512) == \
        m.workspace_size(m.WS_FORWARD, 4096, 256, 8, 2048, 512)
    f = lambda x=FAKE, T=16, nb=1 << 30, layer=lay: L.moe_q4_forward_det(
        x, None, None, FAKE, None, FAKE, T, 8, ctypes.byref(layer), None, FAKE, FAKE, FAKE, FAKE, nb, None, None)
    assert f(T=0) == _lib.OK
    assert f(x=None) == _lib.ERR_INVALID_ARG
    assert f(layer=_layer(fmt=4)) == _lib.ERR_UNSUPPORTED
    assert f(nb=m.workspace_size(m.WS_FORWARD, 16, 256, 8, 2048, 512)) == _lib.ERR_WORKSPACE


def test_dequant_and_residual_validation():
    L = m.lib()
    lay = _layer()
    assert L.moe_q4_dequant(ctypes.byref(lay), 256, 0, FAKE, None) == _lib.ERR_INVALID_ARG
    assert L.moe_q4_dequant(ctypes.byref(lay), 0, 3, FAKE, None) == _lib.ERR_INVALID_ARG
    assert L.moe_q4_dequant(ctypes.byref(lay), 0, 0, None, None) == _lib.ERR_INVALID_ARG
    assert L.moe_q4_residual_bf16(FAKE, FAKE, -1, FAKE, None) == _lib.ERR_INVALID_ARG
    assert L.moe_q4_residual_bf16(FAKE, None, 5, FAKE, None) == _lib.ERR_INVALID_ARG
    assert L.moe_q4_residual_bf16(None, None, 0, None, None) == _lib.OK


def test_python_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, dtype=torch.int16)
    with pytest.raises(ValueError):
        _lib._ptr(x)


def _shared(H=2048, I=512, null=None, misalign=None):
    ptrs = {n: FAKE for n in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s")}
    if null:
        ptrs[null] = None
    if misalign:
        ptrs[misalign] += 2 if misalign.endswith("_q") else 1
    return _lib.SharedExpert(H, I, *[ptrs[n] for n in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s")])


def test_shared_validation():
    L = m.lib()

    def call(sx, T=4, x=FAKE, y=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return L.moe_q4_shared(x, T, ctypes.byref(sx) if sx is not None else None, y, 0, ws, ws_bytes, None)

    assert call(None) == _lib.ERR_INVALID_ARG
    for n in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s"):
        assert call(_shared(null=n)) == _lib.ERR_INVALID_ARG, n
        assert call(_shared(misalign=n)) == _lib.ERR_INVALID_ARG, n
    assert call(_shared(), x=None) == _lib.ERR_INVALID_ARG
    assert call(_shared(), y=None) == _lib.ERR_INVALID_ARG
    assert call(_shared(), x=FAKE + 8) == _lib.ERR_INVALID_ARG
    assert call(_shared(), T=-1) == _lib.ERR_INVALID_ARG
    assert call(_shared(H=0)) == _lib.ERR_INVALID_ARG
    for H, I in ((64, 512), (4096, 512), (2048, 64), (2048, 4096), (1536, 512), (2048, 384)):
        assert call(_shared(H=H, I=I)) == _lib.ERR_UNSUPPORTED, (H, I)
    assert call(_shared(), T=1 << 21) == _lib.ERR_UNSUPPORTED       # T * H >= 2^31
    assert call(_shared(), T=0) == _lib.OK
    need = m.workspace_size(m.WS_SHARED, 4, 1, 1, 2048, 512)
    assert need >= 4 * 512 * 2
    assert call(_shared(), ws_bytes=need - 1) == _lib.ERR_WORKSPACE
    assert call(_shared(), ws=None) == _lib.ERR_WORKSPACE
    ev = (ctypes.c_void_p * 4)(FAKE, FAKE, None, FAKE)
    assert L.moe_q4_shared_timed(FAKE, 4, ctypes.byref(_shared()), FAKE, 0, FAKE, 1 << 30, None,
                                 ev) == _lib.ERR_INVALID_ARG
    assert L.moe_q4_shared_timed(FAKE, 4, ctypes.byref(_shared()), FAKE, 0, FAKE, 1 << 30, None,
                                 None) == _lib.ERR_INVALID_ARG
    assert L.moe_q4_dequant_int8(ctypes.byref(_shared()), 3, FAKE, None) == _lib.ERR_INVALID_ARG
    assert L.moe_q4_dequant_int8(ctypes.byref(_shared()), 0, None, None) == _lib.ERR_INVALID_ARG
    assert L.moe_q4_dequant_int8(ctypes.byref(_shared(I=96)), 0, FAKE, None) == _lib.ERR_UNSUPPORTED


def test_forward_ex_shared_validation():
    L = m.lib()
    lay = _layer()

    def call(sx, T=4, ws_bytes=1 << 30):
        return L.moe_q4_forward_ex(FAKE, None, None, FAKE, None, FAKE, T, 8, ctypes.byref(lay),
                                   ctypes.byref(sx) if sx is not None else None, FAKE, FAKE, FAKE, FAKE, ws_bytes,
                                   None, None)

    assert call(_shared(null="down_s")) == _lib.ERR_INVALID_ARG
    assert call(_shared(H=1024)) == _lib.ERR_INVALID_ARG          # hidden differs from the layer's
    assert call(_shared(I=96)) == _lib.ERR_UNSUPPORTED
    assert call(_shared(), T=0) == _lib.OK
    fwd = m.workspace_size(m.WS_FORWARD, 4, 256, 8, 2048, 512)
    sh = m.workspace_size(m.WS_SHARED, 4, 1, 1, 2048, 1024)
    assert call(_shared(I=1024), ws_bytes=fwd + sh - 1) == _lib.ERR_WORKSPACE
    assert call(None, ws_bytes=fwd - 1) == _lib.ERR_WORKSPACE


def test_fp8_layer_validation():
    """Block-FP8 experts: H, I >= 128 (and the grouped GEMMs' H % 256)."""
    assert _decode(_layer(fmt=2, H=128, I=128), prefill=True) == _lib.ERR_UNSUPPORTED
    assert _decode(_layer(fmt=2), prefill=True, ws_bytes=16) == _lib.ERR_WORKSPACE
    assert _decode(_layer(fmt=2, H=64)) == _lib.ERR_UNSUPPORTED
    assert _decode(_layer(fmt=2, I=64)) == _lib.ERR_UNSUPPORTED
    assert _decode(_layer(fmt=2), T=0) == _lib.OK
    assert _decode(_layer(fmt=4)) == _lib.ERR_UNSUPPORTED
    assert _decode(_layer(fmt=2), ws_bytes=16) == _lib.ERR_WORKSPACE


def test_nvfp4_layer_validation():
    """NVFP4 experts need their global scales (4-byte aligned)."""
    lay = _layer(fmt=3)
    assert _decode(lay) == _lib.ERR_INVALID_ARG          # no global scales
    lay.global_scale = FAKE + 2
    assert _decode(lay) == _lib.ERR_INVALID_ARG          # misaligned
    lay.global_scale = FAKE
    assert _decode(lay, T=0) == _lib.OK
    assert _decode(lay, ws_bytes=16) == _lib.ERR_WORKSPACE
    assert _decode(lay, prefill=True, ws_bytes=16) == _lib.ERR_WORKSPACE
    lay64 = _layer(fmt=3, H=64, I=64)
    lay64.global_scale = FAKE
    assert _decode(lay64, prefill=True) == _lib.ERR_UNSUPPORTED   # grouped GEMMs: H % 256, I % 128


def test_prefill_pack_validation():
    """The prefill copy: its size (27 E I H / 16 bytes, plus a lift byte per
    weight row for int4, a host computation), the formats and shapes it
    takes, and the checks of dst and of the layer's prefill_pack field."""
    lib = m.lib()
    for fmt in (0, 1):
        assert m.moe_q4_prefill_pack_size(_layer(fmt=fmt)) == \
            27 * 256 * 512 * 2048 // 16 + 2 * 256 * 512 + 256 * 2048
    nv = _layer(fmt=3, E=8, H=256, I=128)
    nv.global_scale = FAKE
    assert m.moe_q4_prefill_pack_size(nv) == 27 * 8 * 128 * 256 // 16
    assert m.moe_q4_prefill_pack_size(_layer(fmt=2)) == 3 * 256 * 512 * 2048  # block FP8: codes only
    assert m.moe_q4_prefill_pack_size(_layer(H=64, I=64)) == 0       # not a prefill shape
    assert m.moe_q4_prefill_pack_size(_layer(null="gate_q")) == 0
    lay = _layer()
    need = m.moe_q4_prefill_pack_size(lay)

    def pack(layer, dst=FAKE, nbytes=None):
        return lib.moe_q4_prefill_pack(ctypes.byref(layer), dst, need if nbytes is None else nbytes, None)

    assert pack(lay, dst=None) == _lib.ERR_INVALID_ARG
    assert pack(lay, dst=FAKE + 16) == _lib.ERR_INVALID_ARG       # 256-byte alignment
    assert pack(lay, nbytes=need - 1) == _lib.ERR_INVALID_ARG
    assert pack(_layer(H=64, I=64)) == _lib.ERR_UNSUPPORTED
    assert pack(_layer(null="down_sm")) == _lib.ERR_INVALID_ARG
    # the field itself: 256-byte aligned
    lay.prefill_pack = FAKE + 64
    assert _decode(lay, prefill=True) == _lib.ERR_INVALID_ARG
    assert _decode(lay) == _lib.ERR_INVALID_ARG
    lay.prefill_pack = FAKE
    assert _decode(lay, prefill=True, T=0) == _lib.OK
    assert _decode(lay, prefill=True, ws_bytes=16) == _lib.ERR_WORKSPACE
    fp8 = _layer(fmt=2)
    fp8.prefill_pack = FAKE
    assert _decode(fp8, prefill=True, T=0) == _lib.OK
    assert _decode(fp8, prefill=True, ws_bytes=16) == _lib.ERR_WORKSPACE
