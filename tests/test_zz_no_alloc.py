"""moe_q4_forward_noalloc (the library's own per-GPU workspace) against
moe_q4_forward with a caller workspace, through the C ABI (needs an MI355X).

Three calls in a row on the same device array, each smaller than the one
before: 100 tokens (prefill path), 16 tokens with the residual input of a
layer chain (decode path, one-launch routing), 3 tokens (decode path, routing
in every gate/up workgroup).  Logits, indices and the chain's x_out must be
bit-identical to moe_q4_forward's, gates within 1e-6, y within the output bar
(the decode path adds slot outputs with float atomics).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import synth
from gpu_cases import GATE_RTOL, assert_close

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_expert_amd as m
    m.lib()


def _run(fn_ws, lay, x, rw, T, k, residual_y):
    import quantized_moe_expert_amd as m
    E, H = lay.num_experts, lay.hidden
    lg = torch.empty((T, E), dtype=torch.int16, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    xo = torch.empty_like(x) if residual_y is not None else None
    if fn_ws is None:
        m.moe_q4_forward_noalloc(x, residual_y, xo, rw, None, lg, T, k, lay, idx, gate, y)
    else:
        m.moe_q4_forward(x, residual_y, xo, rw, None, lg, T, k, lay, idx, gate, y, fn_ws)
    torch.cuda.synchronize()
    return lg, idx, gate, y, xo


def test_noalloc_matches_forward_on_successive_calls():
    import quantized_moe_expert_amd as m
    E, H, I, k = 256, 2048, 512, 8
    lay = synth.random_layer(E, H, I, synth.FMT_ASYM_G64, seed=31, device="cuda")
    rw = synth.bf16_bits(synth.normal((E, H), 0.02, 31, "na/w", "cuda"))
    for T, chain in ((100, False), (16, True), (3, False)):
        need = m.workspace_size(m.WS_FORWARD, T, E, k, H, I)
        say(f"[noalloc] T={T} residual={chain} workspace {need} bytes")
        assert need <= m.NOALLOC_SCRATCH_BYTES
        x = synth.bf16_bits(synth.normal((T, H), 1.0, 31, f"na/x/{T}", "cuda"))
        yres = synth.normal((T, H), 0.5, 31, f"na/y/{T}", "cuda") if chain else None
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        m.moe_q4_workspace_init(ws)
        ref = _run(ws, lay, x, rw, T, k, yres)
        got = _run(None, lay, x, rw, T, k, yres)
        assert torch.equal(got[0], ref[0]), "logits differ"
        assert torch.equal(got[1], ref[1]), "expert indices differ"
        assert np.allclose(got[2].cpu().numpy(), ref[2].cpu().numpy(), rtol=GATE_RTOL, atol=0), "gates differ"
        if chain:
            assert torch.equal(got[4], ref[4]), "residual x_out differs"
        r, a = assert_close(got[3].cpu().numpy(), ref[3].cpu().numpy(), f"noalloc T={T}")
        say(f"[noalloc] T={T}: rel L2 {r:.2e} max abs {a:.2e} against moe_q4_forward")
