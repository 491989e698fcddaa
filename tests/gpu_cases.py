"""Shared pieces of the GPU parity tests: run the HIP path, run the oracle,
compare.  Inputs come from the seeded generator only; expected values come
from the oracle only."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import quantized_moe_expert_amd as m

# output tolerance: relative L2 and max abs against the fp64 oracle
REL_L2 = 2e-3
MAX_ABS = 1e-2
GATE_RTOL = 1e-6


def np_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def assert_close(got, ref, what="", abs_scaled=False):
    """rel L2 <= REL_L2 and max abs <= MAX_ABS.  With abs_scaled (inputs far
    from unit scale) the max-abs bound is MAX_ABS times the reference's
    largest magnitude when that exceeds 1: the bound is stated for outputs of
    unit scale, and an output scaled by 2^s carries the same relative
    rounding."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    r = rel_l2(got, ref)
    a = float(np.max(np.abs(got - ref))) if got.size else 0.0
    bound = MAX_ABS * max(1.0, float(np.max(np.abs(ref))) if ref.size else 1.0) if abs_scaled else MAX_ABS
    assert r <= REL_L2 and a <= bound, f"{what}: rel L2 {r:.3e} max abs {a:.3e} (bound {bound:.3e})"
    return r, a


def hip_route(x, router_w, logits, T, H, E, k, bias=None):
    """Returns (logits, idx, gate) from the library; x = None takes logits as given."""
    dev = "cuda"
    lg = torch.empty((T, E), dtype=torch.int16, device=dev) if logits is None else logits.clone()
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    m.moe_q4_route(x, router_w, bias, lg, T, H, E, k, idx, gate)
    return lg, idx, gate


def hip_experts(mode, layer, x, idx, gate, k):
    T = x.shape[0]
    kind = m.WS_DECODE if mode == "decode" else m.WS_PREFILL
    ws = torch.empty(max(m.workspace_size(kind, T, layer.num_experts, k, layer.hidden, layer.inter), 256),
                     dtype=torch.uint8, device="cuda")
    y = torch.full((T, layer.hidden), float("nan"), dtype=torch.float32, device="cuda")
    fn = m.moe_q4_decode if mode == "decode" else m.moe_q4_prefill
    fn(x, idx, gate, T, k, layer, y, ws)
    return y


def oracle_route(case, x_np, tokens=None):
    """Oracle logits/idx/gate for the listed tokens of a case."""
    T, H, E, k = x_np.shape[0], case.H, case.E, case.k
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    if case.router_w is not None:
        lg = oracle.router(np.ascontiguousarray(x_np[tokens]), np_u16(case.router_w), len(tokens), H, E)
    else:
        lg = np.ascontiguousarray(np_u16(case.logits)[tokens])
    idx, gate = oracle.topk(lg, len(tokens), E, k)
    return lg, idx, gate


def oracle_y(layer, x_np, idx, gate, k, tokens=None):
    """Oracle y for tokens (rows of x_np/idx/gate already restricted to them)."""
    n = x_np.shape[0] if tokens is None else len(tokens)
    xs = x_np if tokens is None else np.ascontiguousarray(x_np[tokens])
    return oracle.experts(layer.fmt, layer.num_experts, layer.hidden, layer.inter, *oracle.layer_np(layer),
                          xs, idx, gate, n, k, global_scale=oracle.layer_global(layer))
