"""Plain CPU oracle of the routed int4 MoE expert layer (ctypes wrapper).

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  The library it wraps
(``moe_oracle.c``) shares no code with the HIP library and is built by
``build()`` below with gcc.

Every function takes and returns numpy arrays on the host:
  bf16 values travel as their raw bits in uint16 (or int16) arrays,
  f16 scales/mins likewise, packed nibbles as uint8.

Parity pins: every function here is checked in ``tests/test_oracle.py``
against closed forms, hand-packed cases, brute force or numpy's own float64
routines (see the docstring of each test).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FMT_ASYM_G64 = 0
FMT_SYM_G128 = 1
FMT_FP8_B128 = 2
FMT_NVFP4 = 3

_lib = None


def compile_source(src_path: str, out_path: str) -> str:
    """gcc build of an oracle source (IEEE semantics: no fast-math, no contraction)."""
    tmp = out_path + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                           "-std=c11", "-Wall", "-Wno-unknown-pragmas", src_path, "-o", tmp, "-lm"])
    os.replace(tmp, out_path)
    return out_path


def build(force: bool = True) -> str:
    """Compile liboracle.so next to its source."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


def bind(path: str):
    """Load an oracle shared library at ``path`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int
    lib.oracle_f16_value.restype = ctypes.c_double
    lib.oracle_f16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
    lib.oracle_dequant_global.restype = i32
    lib.oracle_dequant_global.argtypes = [i32, P, P, ctypes.c_float, i32, i32, P]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_bf16_round.restype = ctypes.c_uint16
    lib.oracle_bf16_round.argtypes = [ctypes.c_float]
    lib.oracle_dequant.restype = i32
    lib.oracle_dequant.argtypes = [i32, P, P, i32, i32, P]
    lib.oracle_router.restype = None
    lib.oracle_router.argtypes = [P, P, P, i64, i32, i32, P]
    lib.oracle_topk.restype = None
    lib.oracle_topk.argtypes = [P, i64, i32, i32, P, P]
    lib.oracle_group.restype = i32
    lib.oracle_group.argtypes = [P, i64, i32, i32, P, P, P, P]
    lib.oracle_experts.restype = i32
    lib.oracle_experts.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, i64, i32, P, i64, P, P]
    lib.oracle_dequant_int8.restype = i32
    lib.oracle_dequant_int8.argtypes = [P, P, i32, i32, P]
    lib.oracle_shared.restype = i32
    lib.oracle_shared.argtypes = [i32, i32, P, P, P, P, P, P, P, i64, P, i64, P, P]
    lib.oracle_residual.restype = None
    lib.oracle_residual.argtypes = [P, P, i64, P]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = bind(_LIB)
    return _lib


def set_threads(n: int) -> int:
    """Set the number of OpenMP threads the oracle's parallel loops use (the
    calling thread's setting) and return the previous number."""
    _load()
    gomp = ctypes.CDLL("libgomp.so.1")  # the runtime the oracle links; already loaded
    prev = int(gomp.omp_get_max_threads())
    gomp.omp_set_num_threads(int(n))
    return prev


def use_library(path):
    """Point every function of this module at another build of the oracle
    (``None`` restores the default build); returns the previous binding."""
    global _lib
    prev = _lib
    _lib = bind(path) if path is not None else None
    return prev


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        a = a.view(dtype) if a.dtype.itemsize == np.dtype(dtype).itemsize else a.astype(dtype)
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def f16_value(bits: int) -> float:
    return _load().oracle_f16_value(int(bits) & 0xFFFF)


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(int(bits) & 0xFFFF)


def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(int(code) & 0xF)


def e4m3_value(bits: int) -> float:
    return _load().oracle_e4m3_value(int(bits) & 0xFF)


def _scales(fmt, sm):
    """Scale array as the library takes it: f16 bits, or float32 for fp8."""
    if fmt == FMT_FP8_B128:
        a = np.ascontiguousarray(sm)
        return a if a.dtype == np.float32 else a.astype(np.float32)
    if fmt == FMT_NVFP4:
        return _c(sm, np.uint8)
    return _c(sm, np.uint16)


def bf16_round(f: float) -> int:
    return int(_load().oracle_bf16_round(float(f)))


def bf16_round_array(a) -> np.ndarray:
    """Vector form of bf16_round (through the same C routine, one call per element)."""
    a = np.asarray(a, dtype=np.float32).ravel()
    f = _load().oracle_bf16_round
    return np.array([f(float(v)) for v in a], dtype=np.uint16)


def dequant(fmt: int, q, sm, N: int, K: int, global_scale: float = 1.0) -> np.ndarray:
    """float32 [N][K] from packed uint8 [N][K/2] and f16-bit scales, or (fp8)
    uint8 codes [N][K] and float32 block scales [N/128][K/128], or (NVFP4)
    packed E2M1 [N][K/2], E4M3 block scales [N][K/16] and the matrix's global
    scale (see moe_oracle.c)."""
    q = _c(q, np.uint8)
    sm = _scales(fmt, sm)
    out = np.empty((N, K), dtype=np.float32)
    rc = _load().oracle_dequant_global(int(fmt), _p(q), _p(sm), float(global_scale), int(N), int(K), _p(out))
    if rc != 0:
        raise ValueError("oracle_dequant: unsupported format or shape")
    return out


def router(x, wr, T: int, H: int, E: int, bias=None) -> np.ndarray:
    """bf16 bits [T][E] of the router logits."""
    x = _c(x, np.uint16)
    wr = _c(wr, np.uint16)
    b = _c(bias, np.float32) if bias is not None else None
    out = np.empty((T, E), dtype=np.uint16)
    _load().oracle_router(_p(x), _p(wr), _p(b), int(T), int(H), int(E), _p(out))
    return out


def topk(logits, T: int, E: int, k: int):
    """(idx int32 [T][k], gate float32 [T][k])."""
    lg = _c(logits, np.uint16)
    idx = np.empty((T, k), dtype=np.int32)
    gate = np.empty((T, k), dtype=np.float32)
    _load().oracle_topk(_p(lg), int(T), int(E), int(k), _p(idx), _p(gate))
    return idx, gate


def group(idx, T: int, k: int, E: int):
    """(cnt [E], off [E+1], perm [T*k], inv [T*k]) int32 of the stable grouping by expert."""
    idx = _c(idx, np.int32)
    cnt = np.empty(E, dtype=np.int32)
    off = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(T * k, dtype=np.int32)
    inv = np.empty(T * k, dtype=np.int32)
    rc = _load().oracle_group(_p(idx), int(T), int(k), int(E), _p(cnt), _p(off), _p(perm), _p(inv))
    if rc != 0:
        raise ValueError("oracle_group: expert index out of range")
    return cnt, off, perm, inv


def experts(fmt, E, H, I, gate_q, up_q, down_q, gate_sm, up_sm, down_sm,
            x, idx, gate, T: int, k: int, tokens=None, global_scale=None) -> np.ndarray:
    """float32 y [ntok][H] for the listed tokens (all T when ``tokens`` is None);
    ``global_scale``: NVFP4 float32 [E][2] = {gate and up, down}."""
    arrs = [_c(a, np.uint8) for a in (gate_q, up_q, down_q)]
    sms = [_scales(fmt, a) for a in (gate_sm, up_sm, down_sm)]
    x = _c(x, np.uint16)
    idx = _c(idx, np.int32)
    gate = _c(gate, np.float32)
    tok = _c(np.asarray(tokens, dtype=np.int64), np.int64) if tokens is not None else None
    ntok = len(tok) if tok is not None else T
    gs = np.ascontiguousarray(global_scale, dtype=np.float32) if global_scale is not None else None
    y = np.empty((ntok, H), dtype=np.float32)
    rc = _load().oracle_experts(int(fmt), int(E), int(H), int(I), *[_p(a) for a in arrs],
                                *[_p(a) for a in sms], _p(x), _p(idx), _p(gate), int(T), int(k),
                                _p(tok), int(ntok), _p(y), _p(gs))
    if rc != 0:
        raise ValueError(f"oracle_experts failed ({rc})")
    return y


def dequant_int8(q, s, N: int, K: int) -> np.ndarray:
    """float32 [N][K] from int8 codes [N][K] and f16-bit scales [N][K/128]."""
    q = _c(q, np.int8)
    s = _c(s, np.uint16)
    out = np.empty((N, K), dtype=np.float32)
    rc = _load().oracle_dequant_int8(_p(q), _p(s), int(N), int(K), _p(out))
    if rc != 0:
        raise ValueError("oracle_dequant_int8: unsupported shape")
    return out


def shared(H, I, gate_q, up_q, down_q, gate_s, up_s, down_s, x, T: int,
           tokens=None, y_in=None) -> np.ndarray:
    """float32 [ntok][H]: y_in (or 0) plus the shared expert's output for the
    listed tokens (all T when ``tokens`` is None)."""
    qs = [_c(a, np.int8) for a in (gate_q, up_q, down_q)]
    ss = [_c(a, np.uint16) for a in (gate_s, up_s, down_s)]
    x = _c(x, np.uint16)
    tok = _c(np.asarray(tokens, dtype=np.int64), np.int64) if tokens is not None else None
    ntok = len(tok) if tok is not None else T
    yi = _c(y_in, np.float32) if y_in is not None else None
    if yi is not None and yi.size != ntok * H:
        raise ValueError("shared: y_in must hold ntok * H values")
    y = np.empty((ntok, H), dtype=np.float32)
    rc = _load().oracle_shared(int(H), int(I), *[_p(a) for a in qs], *[_p(a) for a in ss],
                               _p(x), int(T), _p(tok), int(ntok), _p(yi), _p(y))
    if rc != 0:
        raise ValueError(f"oracle_shared failed ({rc})")
    return y


def residual(x, y) -> np.ndarray:
    """bf16 bits of bf16(float(x) + y), elementwise."""
    x = _c(x, np.uint16)
    y = _c(y, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_residual(_p(x), _p(y), int(x.size), _p(out))
    return out


def layer_np(layer):
    """numpy views of a synth.Layer's tensors (moved to the host)."""
    return [t.cpu().numpy() for t in (layer.gate_q, layer.up_q, layer.down_q,
                                      layer.gate_sm, layer.up_sm, layer.down_sm)]


def layer_global(layer):
    """NVFP4 global scales of a synth.Layer (host float32 [E][2]) or None."""
    g = getattr(layer, "global_scale", None)
    return g.cpu().numpy() if g is not None else None


def moe_layer(layer, x, T, k, router_w=None, logits=None, bias=None, tokens=None):
    """Whole layer for the listed tokens: returns (logits, idx, gate, y) of those tokens.

    ``router_w`` (bf16 bits [E][H]) computes the logits; otherwise ``logits``
    (bf16 bits [T][E]) are taken as given.
    """
    E, H, I = layer.num_experts, layer.hidden, layer.inter
    x = np.asarray(x).view(np.uint16).reshape(T, H)
    if tokens is None:
        tokens = np.arange(T, dtype=np.int64)
    tokens = np.asarray(tokens, dtype=np.int64)
    xs = np.ascontiguousarray(x[tokens])
    n = len(tokens)
    if router_w is not None:
        lg = router(xs, np.asarray(router_w).view(np.uint16), n, H, E, bias)
    else:
        lg = np.ascontiguousarray(np.asarray(logits).view(np.uint16).reshape(T, E)[tokens])
    idx, gate = topk(lg, n, E, k)
    y = experts(layer.fmt, E, H, I, *layer_np(layer), xs, idx, gate, n, k, global_scale=layer_global(layer))
    return lg, idx, gate, y
