"""ctypes binding of libmoe_q4.so with the C ABI's names.

Argument marshalling only: tensors are passed as device pointers
(``tensor.data_ptr()``) and the stream as torch's current HIP stream.  Every
step of the layer runs in the library's HIP kernels; there is no fallback, and
loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_q4.so")

ASYM_G64 = 0
SYM_G128 = 1
FP8_B128 = 2
NVFP4 = 3
WS_ROUTE, WS_DECODE, WS_PREFILL, WS_GROUP, WS_FORWARD, WS_SHARED, WS_FORWARD_DET = 0, 1, 2, 3, 4, 5, 6
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4

# every entry point declared in include/moe_q4.h
EXPORTS = ("moe_q4_workspace_size", "moe_q4_route", "moe_q4_group", "moe_q4_decode", "moe_q4_prefill",
           "moe_q4_decode_timed", "moe_q4_prefill_timed", "moe_q4_forward", "moe_q4_forward_timed",
           "moe_q4_workspace_init",
           "moe_q4_shared", "moe_q4_shared_timed", "moe_q4_dequant_int8", "moe_q4_forward_ex",
           "moe_q4_dequant", "moe_q4_residual_bf16", "moe_q4_error_string",
           "moe_q4_prefill_pack_size", "moe_q4_prefill_pack", "moe_q4_forward_noalloc", "moe_q4_forward_det",
           "moe_q4_frame_workspace_size", "moe_q4_frame")
NOALLOC_SCRATCH_BYTES = 16 << 20  # MOE_Q4_NOALLOC_SCRATCH_BYTES
STAGE_EVENTS = 4
FRAME_MAX_LANES = 4  # MOE_Q4_FRAME_MAX_LANES


class MoeQ4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({error_string(status)})")
        self.status = status


class Layer(ctypes.Structure):
    """struct moe_q4_layer"""
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("format", ctypes.c_int32),
                ("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p), ("down_q", ctypes.c_void_p),
                ("gate_sm", ctypes.c_void_p), ("up_sm", ctypes.c_void_p), ("down_sm", ctypes.c_void_p),
                ("global_scale", ctypes.c_void_p), ("prefill_pack", ctypes.c_void_p)]


class SharedExpert(ctypes.Structure):
    """struct moe_q4_shared_expert"""
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p), ("down_q", ctypes.c_void_p),
                ("gate_s", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m quantized_moe_expert_amd.build` "
                              "(or __graft_entry__.build())")
        import torch  # noqa: F401  (load torch's HIP runtime first: one runtime per process)
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.moe_q4_workspace_size.restype = sz
        L.moe_q4_workspace_size.argtypes = [ctypes.c_int, i64, i32, i32, i32, i32]
        L.moe_q4_route.restype = ctypes.c_int
        L.moe_q4_route.argtypes = [P, P, P, P, i64, i32, i32, i32, P, P, P, sz, P]
        L.moe_q4_group.restype = ctypes.c_int
        L.moe_q4_group.argtypes = [P, i64, i32, i32, P, P, P, P, P, sz, P]
        for name in ("moe_q4_decode", "moe_q4_prefill"):
            fn = getattr(L, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [P, P, P, i64, i32, ctypes.POINTER(Layer), P, P, sz, P]
        for name in ("moe_q4_decode_timed", "moe_q4_prefill_timed"):
            fn = getattr(L, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [P, P, P, i64, i32, ctypes.POINTER(Layer), P, P, sz, P, ctypes.POINTER(ctypes.c_void_p)]
        L.moe_q4_forward.restype = ctypes.c_int
        L.moe_q4_forward.argtypes = [P, P, P, P, P, P, i64, i32, ctypes.POINTER(Layer), P, P, P, P, sz, P]
        L.moe_q4_forward_noalloc.restype = ctypes.c_int
        L.moe_q4_forward_noalloc.argtypes = [P, P, P, P, P, P, i64, i32, ctypes.POINTER(Layer), P, P, P, P]
        L.moe_q4_forward_timed.restype = ctypes.c_int
        L.moe_q4_forward_timed.argtypes = [P, P, P, P, P, P, i64, i32, ctypes.POINTER(Layer), P, P, P, P, sz, P,
                                           ctypes.POINTER(ctypes.c_void_p)]
        L.moe_q4_forward_ex.restype = ctypes.c_int
        L.moe_q4_forward_ex.argtypes = [P, P, P, P, P, P, i64, i32, ctypes.POINTER(Layer),
                                        ctypes.POINTER(SharedExpert), P, P, P, P, sz, P,
                                        ctypes.POINTER(ctypes.c_void_p)]
        L.moe_q4_forward_det.restype = ctypes.c_int
        L.moe_q4_forward_det.argtypes = L.moe_q4_forward_ex.argtypes
        L.moe_q4_frame_workspace_size.restype = sz
        L.moe_q4_frame_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32, i32]
        L.moe_q4_frame.restype = ctypes.c_int
        L.moe_q4_frame.argtypes = [P, i64, i32, i32, ctypes.POINTER(Layer), ctypes.POINTER(ctypes.c_void_p),
                                   ctypes.POINTER(SharedExpert), P, P, P, P, P, i32,
                                   ctypes.POINTER(ctypes.c_void_p), P, sz, ctypes.POINTER(ctypes.c_void_p)]
        L.moe_q4_workspace_init.restype = ctypes.c_int
        L.moe_q4_workspace_init.argtypes = [P, sz, P]
        L.moe_q4_dequant.restype = ctypes.c_int
        L.moe_q4_dequant.argtypes = [ctypes.POINTER(Layer), i32, i32, P, P]
        L.moe_q4_shared.restype = ctypes.c_int
        L.moe_q4_shared.argtypes = [P, i64, ctypes.POINTER(SharedExpert), P, i32, P, sz, P]
        L.moe_q4_shared_timed.restype = ctypes.c_int
        L.moe_q4_shared_timed.argtypes = [P, i64, ctypes.POINTER(SharedExpert), P, i32, P, sz, P,
                                          ctypes.POINTER(ctypes.c_void_p)]
        L.moe_q4_dequant_int8.restype = ctypes.c_int
        L.moe_q4_dequant_int8.argtypes = [ctypes.POINTER(SharedExpert), i32, P, P]
        L.moe_q4_residual_bf16.restype = ctypes.c_int
        L.moe_q4_residual_bf16.argtypes = [P, P, i64, P, P]
        L.moe_q4_prefill_pack_size.restype = sz
        L.moe_q4_prefill_pack_size.argtypes = [ctypes.POINTER(Layer)]
        L.moe_q4_prefill_pack.restype = ctypes.c_int
        L.moe_q4_prefill_pack.argtypes = [ctypes.POINTER(Layer), P, sz, P]
        L.moe_q4_error_string.restype = ctypes.c_char_p
        L.moe_q4_error_string.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def error_string(status: int) -> str:
    return lib().moe_q4_error_string(int(status)).decode()


def _ptr(t):
    """Device pointer of a tensor (None -> NULL).  Plain ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("moe_q4 takes device tensors")
    if not t.is_contiguous():
        raise ValueError("moe_q4 takes contiguous tensors")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != OK:
        raise MoeQ4Error(fn, status)


def layer_struct(layer, pack=None) -> Layer:
    """struct moe_q4_layer from an object with num_experts, hidden, inter, fmt
    (or format) and the six gate/up/down code and scale tensors; ``pack``:
    the layer's prefill copy (uint8 device tensor from prefill_pack) or None."""
    fmt = getattr(layer, "fmt", None)
    if fmt is None:
        fmt = layer.format
    return Layer(int(layer.num_experts), int(layer.hidden), int(layer.inter), int(fmt),
                 _ptr(layer.gate_q), _ptr(layer.up_q), _ptr(layer.down_q),
                 _ptr(layer.gate_sm), _ptr(layer.up_sm), _ptr(layer.down_sm),
                 _ptr(getattr(layer, "global_scale", None)), _ptr(pack))


def shared_struct(sx) -> SharedExpert:
    """struct moe_q4_shared_expert from an object with hidden, inter and the six
    gate/up/down code (int8) and scale (f16 bits) tensors."""
    return SharedExpert(int(sx.hidden), int(sx.inter), _ptr(sx.gate_q), _ptr(sx.up_q), _ptr(sx.down_q),
                        _ptr(sx.gate_s), _ptr(sx.up_s), _ptr(sx.down_s))


def workspace_size(kind: int, T: int, E: int, k: int, H: int, I: int) -> int:
    return int(lib().moe_q4_workspace_size(int(kind), int(T), int(E), int(k), int(H), int(I)))


def _ws(ws):
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


def moe_q4_route(x, router_w, bias, logits, T, H, E, k, topk_idx, topk_gate, ws=None, stream=None):
    w, nb = _ws(ws)
    _check("moe_q4_route", lib().moe_q4_route(_ptr(x), _ptr(router_w), _ptr(bias), _ptr(logits), T, H, E, k,
                                               _ptr(topk_idx), _ptr(topk_gate), w, nb, _stream(stream)))


def moe_q4_group(topk_idx, T, k, E, cnt, off, perm, inv, ws, stream=None):
    w, nb = _ws(ws)
    _check("moe_q4_group", lib().moe_q4_group(_ptr(topk_idx), T, k, E, _ptr(cnt), _ptr(off), _ptr(perm),
                                               _ptr(inv), w, nb, _stream(stream)))


def moe_q4_decode(x, topk_idx, topk_gate, T, k, layer, y, ws, stream=None):
    w, nb = _ws(ws)
    st = layer_struct(layer) if not isinstance(layer, Layer) else layer
    _check("moe_q4_decode", lib().moe_q4_decode(_ptr(x), _ptr(topk_idx), _ptr(topk_gate), T, k,
                                                 ctypes.byref(st), _ptr(y), w, nb, _stream(stream)))


def moe_q4_prefill(x, topk_idx, topk_gate, T, k, layer, y, ws, stream=None):
    w, nb = _ws(ws)
    st = layer_struct(layer) if not isinstance(layer, Layer) else layer
    _check("moe_q4_prefill", lib().moe_q4_prefill(_ptr(x), _ptr(topk_idx), _ptr(topk_gate), T, k,
                                                   ctypes.byref(st), _ptr(y), w, nb, _stream(stream)))


def _timed(name, x, topk_idx, topk_gate, T, k, layer, y, ws, events, stream):
    w, nb = _ws(ws)
    st = layer_struct(layer) if not isinstance(layer, Layer) else layer
    ev = (ctypes.c_void_p * STAGE_EVENTS)(*[int(e) for e in events])
    _check(name, getattr(lib(), name)(_ptr(x), _ptr(topk_idx), _ptr(topk_gate), T, k, ctypes.byref(st), _ptr(y),
                                      w, nb, _stream(stream), ev))


def moe_q4_decode_timed(x, topk_idx, topk_gate, T, k, layer, y, ws, events, stream=None):
    """moe_q4_decode that has the runtime record the 4 given hipEvent_t handles at the start and end
    of its gate/up GEMV kernel ([0], [1]) and grouping kernel ([2], [3])."""
    _timed("moe_q4_decode_timed", x, topk_idx, topk_gate, T, k, layer, y, ws, events, stream)


def moe_q4_prefill_timed(x, topk_idx, topk_gate, T, k, layer, y, ws, events, stream=None):
    _timed("moe_q4_prefill_timed", x, topk_idx, topk_gate, T, k, layer, y, ws, events, stream)


def moe_q4_forward_timed(x, residual_y, x_out, router_w, bias, logits, T, k, layer, topk_idx, topk_gate, y, ws,
                         events, stream=None):
    """moe_q4_forward that has the runtime record the 4 given hipEvent_t handles around its two main
    kernels: decode [0], [1] gate/up GEMV and [2], [3] routing; prefill [0], [1] gate/up GEMM and [2], [3]
    down GEMM."""
    w, nb = _ws(ws)
    st = layer_struct(layer) if not isinstance(layer, Layer) else layer
    ev = (ctypes.c_void_p * STAGE_EVENTS)(*[int(e) for e in events])
    _check("moe_q4_forward_timed",
           lib().moe_q4_forward_timed(_ptr(x), _ptr(residual_y), _ptr(x_out), _ptr(router_w), _ptr(bias),
                                      _ptr(logits), T, k, ctypes.byref(st), _ptr(topk_idx), _ptr(topk_gate),
                                      _ptr(y), w, nb, _stream(stream), ev))


def moe_q4_forward(x, residual_y, x_out, router_w, bias, logits, T, k, layer, topk_idx, topk_gate, y, ws,
                   stream=None):
    w, nb = _ws(ws)
    st = layer_struct(layer) if not isinstance(layer, Layer) else layer
    _check("moe_q4_forward", lib().moe_q4_forward(_ptr(x), _ptr(residual_y), _ptr(x_out), _ptr(router_w), _ptr(bias),
                                                   _ptr(logits), T, k, ctypes.byref(st), _ptr(topk_idx),
                                                   _ptr(topk_gate), _ptr(y), w, nb, _stream(stream)))


def moe_q4_forward_noalloc(x, residual_y, x_out, router_w, bias, logits, T, k, layer, topk_idx, topk_gate, y,
                           stream=None):
    """moe_q4_forward on the library's own per-GPU device array (no workspace argument)."""
    st = layer_struct(layer) if not isinstance(layer, Layer) else layer
    _check("moe_q4_forward_noalloc",
           lib().moe_q4_forward_noalloc(_ptr(x), _ptr(residual_y), _ptr(x_out), _ptr(router_w), _ptr(bias),
                                        _ptr(logits), T, k, ctypes.byref(st), _ptr(topk_idx), _ptr(topk_gate),
                                        _ptr(y), _stream(stream)))


def moe_q4_forward_ex(x, residual_y, x_out, router_w, bias, logits, T, k, layer, shared, topk_idx, topk_gate, y,
                      ws, stream=None, events=None, _name="moe_q4_forward_ex"):
    """moe_q4_forward with the layer's shared expert (None: without); ``events``: None or 4 hipEvent_t
    handles as moe_q4_forward_timed."""
    w, nb = _ws(ws)
    st = layer_struct(layer) if not isinstance(layer, Layer) else layer
    sx = None
    if shared is not None:
        sx = ctypes.byref(shared_struct(shared) if not isinstance(shared, SharedExpert) else shared)
    ev = (ctypes.c_void_p * STAGE_EVENTS)(*[int(e) for e in events]) if events is not None else None
    _check(_name,
           getattr(lib(), _name)(_ptr(x), _ptr(residual_y), _ptr(x_out), _ptr(router_w), _ptr(bias), _ptr(logits),
                                 T, k, ctypes.byref(st), sx, _ptr(topk_idx), _ptr(topk_gate), _ptr(y), w, nb,
                                 _stream(stream), ev))


def moe_q4_forward_det(x, residual_y, x_out, router_w, bias, logits, T, k, layer, shared, topk_idx, topk_gate, y,
                       ws, stream=None, events=None):
    """moe_q4_forward_ex with a run-to-run identical decode y (routed rows summed in slot order); the
    workspace from workspace_size(WS_FORWARD_DET, ...)."""
    moe_q4_forward_ex(x, residual_y, x_out, router_w, bias, logits, T, k, layer, shared, topk_idx, topk_gate, y,
                      ws, stream, events, _name="moe_q4_forward_det")


def frame_workspace_size(T: int, E: int, k: int, H: int, I: int, shared_inter: int, lanes: int) -> int:
    return int(lib().moe_q4_frame_workspace_size(int(T), int(E), int(k), int(H), int(I), int(shared_inter),
                                                 int(lanes)))


def moe_q4_frame(x, T, k, layers, routers, shared, x_chain, y_chain, logits, topk_idx, topk_gate, lanes, streams,
                 ws, events=None):
    """A decode frame of len(layers) layers as ``lanes`` token lanes, lane i on streams[i] (torch streams or
    raw handles); ``layers`` / ``shared``: lists of Layer / SharedExpert structs (or objects with their
    tensors), ``shared`` None for none; ``events``: None or len(layers) * lanes * STAGE_EVENTS handles."""
    n = len(layers)
    lay = (Layer * n)(*[l if isinstance(l, Layer) else layer_struct(l) for l in layers])
    rws = (ctypes.c_void_p * n)(*[_ptr(r) for r in routers])
    sx = None
    if shared is not None:
        sx = (SharedExpert * n)(*[s if isinstance(s, SharedExpert) else shared_struct(s) for s in shared])
    sts = (ctypes.c_void_p * len(streams))(*[_stream(s) for s in streams])
    ev = (ctypes.c_void_p * len(events))(*[int(e) for e in events]) if events is not None else None
    w, nb = _ws(ws)
    _check("moe_q4_frame",
           lib().moe_q4_frame(_ptr(x), T, k, n, lay, rws, sx, _ptr(x_chain), _ptr(y_chain), _ptr(logits),
                              _ptr(topk_idx), _ptr(topk_gate), lanes, sts, w, nb, ev))


def moe_q4_workspace_init(ws, stream=None):
    w, nb = _ws(ws)
    _check("moe_q4_workspace_init", lib().moe_q4_workspace_init(w, nb, _stream(stream)))


def moe_q4_dequant(layer, expert, proj, out, stream=None):
    st = layer_struct(layer) if not isinstance(layer, Layer) else layer
    _check("moe_q4_dequant", lib().moe_q4_dequant(ctypes.byref(st), expert, proj, _ptr(out), _stream(stream)))


def moe_q4_prefill_pack_size(layer) -> int:
    st = layer_struct(layer) if not isinstance(layer, Layer) else layer
    return int(lib().moe_q4_prefill_pack_size(ctypes.byref(st)))


def moe_q4_prefill_pack(layer, dst, stream=None):
    """Writes the layer's prefill copy into ``dst`` (uint8 device tensor of at
    least moe_q4_prefill_pack_size bytes, 256-byte aligned)."""
    st = layer_struct(layer) if not isinstance(layer, Layer) else layer
    nb = 0 if dst is None else dst.numel() * dst.element_size()
    _check("moe_q4_prefill_pack", lib().moe_q4_prefill_pack(ctypes.byref(st), _ptr(dst), nb, _stream(stream)))


def prefill_pack(layer, device="cuda", stream=None):
    """Allocates and fills the layer's prefill copy; returns the uint8 tensor
    (pass it to layer_struct(layer, pack=...))."""
    import torch
    n = moe_q4_prefill_pack_size(layer)
    if n == 0:
        raise MoeQ4Error("moe_q4_prefill_pack_size", -2)
    dst = torch.empty(n, dtype=torch.uint8, device=device)
    moe_q4_prefill_pack(layer, dst, stream)
    return dst


def moe_q4_residual_bf16(x, y, n, out, stream=None):
    _check("moe_q4_residual_bf16", lib().moe_q4_residual_bf16(_ptr(x), _ptr(y), n, _ptr(out), _stream(stream)))


def moe_q4_shared(x, T, shared, y, accumulate, ws, stream=None):
    w, nb = _ws(ws)
    st = shared_struct(shared) if not isinstance(shared, SharedExpert) else shared
    _check("moe_q4_shared", lib().moe_q4_shared(_ptr(x), T, ctypes.byref(st), _ptr(y), int(bool(accumulate)), w, nb,
                                                 _stream(stream)))


def moe_q4_shared_timed(x, T, shared, y, accumulate, ws, events, stream=None):
    """moe_q4_shared that has the runtime record the 4 given hipEvent_t handles at the start and end of its
    gate/up launch ([0], [1]) and its down launch ([2], [3])."""
    w, nb = _ws(ws)
    st = shared_struct(shared) if not isinstance(shared, SharedExpert) else shared
    ev = (ctypes.c_void_p * STAGE_EVENTS)(*[int(e) for e in events])
    _check("moe_q4_shared_timed", lib().moe_q4_shared_timed(_ptr(x), T, ctypes.byref(st), _ptr(y),
                                                             int(bool(accumulate)), w, nb, _stream(stream), ev))


def moe_q4_dequant_int8(shared, proj, out, stream=None):
    st = shared_struct(shared) if not isinstance(shared, SharedExpert) else shared
    _check("moe_q4_dequant_int8", lib().moe_q4_dequant_int8(ctypes.byref(st), proj, _ptr(out), _stream(stream)))
