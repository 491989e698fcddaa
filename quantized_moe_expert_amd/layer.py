"""Convenience wrapper: buffers for one routed int4 MoE layer call.

Allocates the outputs and the workspace once (torch device memory) and calls
the C ABI; the computation itself is the library's.
"""
from __future__ import annotations

import torch

from . import _lib


class MoeQ4Layer:
    """Route + expert layer for batches of up to ``max_tokens`` tokens.

    ``weights``: object with num_experts, hidden, inter, fmt and the six
    device tensors gate_q, up_q, down_q, gate_sm, up_sm, down_sm (canonical
    layout of include/moe_q4.h).  ``mode``: "decode" (GEMV path) or
    "prefill" (grouped-GEMM path).  ``shared``: the layer's shared expert
    (hidden, inter and the six int8 code / f16 scale tensors) or None;
    forward() then adds its output to every token's.  ``pack_prefill``: make
    the prefill copy of the weights, which the prefill GEMMs then read.
    """

    def __init__(self, weights, k: int, max_tokens: int, mode: str = "decode", device="cuda", shared=None,
                 pack_prefill: bool = False):
        if mode not in ("decode", "prefill"):
            raise ValueError("mode must be 'decode' or 'prefill'")
        self.w = weights
        self.k = k
        self.E, self.H, self.I = weights.num_experts, weights.hidden, weights.inter
        self.mode = mode
        self.max_tokens = max_tokens
        self.pack = _lib.prefill_pack(weights, device) if pack_prefill else None
        self.struct = _lib.layer_struct(weights, pack=self.pack)
        T = max_tokens
        kind = _lib.WS_DECODE if mode == "decode" else _lib.WS_PREFILL
        nbytes = max(_lib.workspace_size(kind, T, self.E, k, self.H, self.I), 256)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.shared = _lib.shared_struct(shared) if shared is not None else None
        self._shared_obj = shared
        fbytes = _lib.workspace_size(_lib.WS_FORWARD, T, self.E, k, self.H, self.I)
        if shared is not None:
            fbytes += _lib.workspace_size(_lib.WS_SHARED, T, 1, 1, self.H, shared.inter)
        fbytes = max(fbytes, 256)
        self.ws_forward = torch.zeros(fbytes, dtype=torch.uint8, device=device)
        _lib.moe_q4_workspace_init(self.ws_forward)
        self.logits = torch.empty((T, self.E), dtype=torch.int16, device=device)
        self.idx = torch.empty((T, k), dtype=torch.int32, device=device)
        self.gate = torch.empty((T, k), dtype=torch.float32, device=device)
        self.y = torch.empty((T, self.H), dtype=torch.float32, device=device)

    def route(self, x=None, router_w=None, logits=None, bias=None, T=None):
        """bf16 logits (computed from x and router_w, or copied from ``logits``)
        -> top-k indices and gates; returns (logits, idx, gate) views."""
        T = x.shape[0] if x is not None else (logits.shape[0] if T is None else T)
        lg = self.logits[:T]
        if x is None:
            lg.copy_(logits)
        _lib.moe_q4_route(x, router_w, bias, lg, T, self.H, self.E, self.k, self.idx[:T], self.gate[:T])
        return lg, self.idx[:T], self.gate[:T]

    def experts(self, x, idx, gate, y=None):
        T = x.shape[0]
        y = self.y[:T] if y is None else y
        fn = _lib.moe_q4_decode if self.mode == "decode" else _lib.moe_q4_prefill
        fn(x, idx, gate, T, self.k, self.struct, y, self.ws)
        return y

    def forward(self, x, router_w=None, logits=None, bias=None, residual_y=None, x_out=None):
        """Whole layer through moe_q4_forward (decode path for <= 64 tokens,
        prefill path above); ``logits`` are used when ``router_w`` is None."""
        T = x.shape[0]
        lg = self.logits[:T]
        if router_w is None:
            lg.copy_(logits)
        y = self.y[:T]
        _lib.moe_q4_forward_ex(x, residual_y, x_out, router_w, bias, lg, T, self.k, self.struct, self.shared,
                               self.idx[:T], self.gate[:T], y, self.ws_forward)
        return y
