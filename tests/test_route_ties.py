"""Signed zeros and NaN / -inf exactly at the k-th place, on every routing path
(needs an MI355X).

-0 equals +0 and a NaN logit ranks as -inf, so both are ties, and ties go to
the lower expert index.  Each token's logits hold k - L distinct leaders
(L = 1..3), then a run of tied values that straddles rank k (a mix of -0 and
+0, or a mix of NaN bit patterns and -inf), then smaller values; some tokens
also put NaNs at low expert indices that must not be chosen.  Indices must
equal the oracle's bit for bit and gates within 1e-6 (a selected NaN / -inf
slot has gate 0).  The routing paths with the logits given:
  - moe_q4_route without x: the top-k launch;
  - moe_q4_forward at 6 tokens x top-8: every gate/up workgroup routes;
  - moe_q4_forward at 16 tokens: the one-launch routing's last workgroup;
  - moe_q4_forward at 100 tokens (800 pairs): prefill with the top-k launch;
  - moe_q4_forward at 200 tokens (1600 pairs): the prefill preparation launch.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import GATE_RTOL, assert_close, hip_route, np_u16, oracle_y
from tie_cases import tie_logits

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_expert_amd as m
    m.lib()


def _check_idx_gate(idx, gate, ir, gr):
    got = idx.cpu().numpy()
    bad = np.argwhere(np.any(got != ir, axis=1)).ravel()
    assert bad.size == 0, f"tokens {bad[:8].tolist()}: got {got[bad[0]].tolist()}, oracle {ir[bad[0]].tolist()}"
    g = gate.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g))
    assert np.array_equal(g == 0, gr == 0), "zero gates differ"
    assert np.allclose(g, gr, rtol=GATE_RTOL, atol=0)


@pytest.mark.parametrize("T,E,k", [(300, 256, 8), (40, 16, 2), (9, 9, 5)])
def test_topk_launch_ties(T, E, k):
    say(f"[ties route] T={T} E={E} k={k}")
    lg = tie_logits(T, E, k, seed=T + E)
    lg_t = torch.from_numpy(lg.view(np.int16).copy()).cuda()
    _, idx, gate = hip_route(None, None, lg_t, T, 0, E, k)
    ir, gr = oracle.topk(lg, T, E, k)
    _check_idx_gate(idx, gate, ir, gr)


@pytest.mark.parametrize("T", [6, 16, 100, 200])
def test_forward_routing_paths_ties(T):
    import quantized_moe_expert_amd as m
    E, H, I, k = 256, 512, 256, 8
    say(f"[ties forward] T={T}")
    lay = synth.random_layer(E, H, I, synth.FMT_ASYM_G64, seed=21, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 21, f"ties/x/{T}", "cuda"))
    lg = tie_logits(T, E, k, seed=T)
    lg_t = torch.from_numpy(lg.view(np.int16).copy()).cuda()
    ws = torch.zeros(max(m.workspace_size(m.WS_FORWARD, T, E, k, H, I), 256), dtype=torch.uint8, device="cuda")
    m.moe_q4_workspace_init(ws)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    m.moe_q4_forward(x, None, None, None, None, lg_t, T, k, lay, idx, gate, y, ws)
    torch.cuda.synchronize()
    ir, gr = oracle.topk(lg, T, E, k)
    _check_idx_gate(idx, gate, ir, gr)
    assert_close(y.cpu().numpy(), oracle_y(lay, np_u16(x), ir, gr, k), f"ties forward T={T}")
