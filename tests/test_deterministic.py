"""The slot-ordered decode entry point moe_q4_forward_det (needs an MI355X).

moe_q4_forward adds each routed row into y with float atomics, so two runs
agree to rounding only.  moe_q4_forward_det stores the routed rows and sums a
token's k rows in slot order: y must be the same bits on every run, within
the float tolerance of the oracle (drama-rs page, "Tests": every kernel
checked against a plain reference), and within rounding of moe_q4_forward.
Cases: the three decode weight formats, both decode routing variants (4
tokens route in every expert workgroup, 16 in the routing launch), a shared
expert (run after the sum), a residual chain step, and a three-layer chain
fed from its own outputs.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import assert_close, np_u16

pytestmark = pytest.mark.gpu

RUNS = 4


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_expert_amd as m
    m.lib()


def _ws(kind, T, E, k, H, I, sx=None):
    import quantized_moe_expert_amd as m
    nb = m.workspace_size(kind, T, E, k, H, I)
    if sx is not None:
        nb += m.workspace_size(m.WS_SHARED, T, 1, 1, H, sx.inter)
    ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device="cuda")
    m.moe_q4_workspace_init(ws)
    return ws


def _run(det, lay, x, rw, T, k, sx=None, residual_y=None, ws=None):
    import quantized_moe_expert_amd as m
    E, H, I = lay.num_experts, lay.hidden, lay.inter
    if ws is None:
        ws = _ws(m.WS_FORWARD_DET if det else m.WS_FORWARD, T, E, k, H, I, sx)
    lg = torch.empty((T, E), dtype=torch.int16, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    xo = torch.empty_like(x) if residual_y is not None else None
    fn = m.moe_q4_forward_det if det else m.moe_q4_forward_ex
    fn(x, residual_y, xo, rw, None, lg, T, k, lay, sx, idx, gate, y, ws)
    torch.cuda.synchronize()
    return y, idx, xo


def _layer_case(fmt, T, seed):
    E, H, I, k = 256, 2048, 512, 8
    lay = synth.random_layer(E, H, I, fmt, seed=seed, device="cuda", tag=f"det/{fmt}")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, seed, f"det/x/{T}", "cuda"))
    rw = synth.bf16_bits(synth.normal((E, H), 0.02, seed, f"det/rw", "cuda"))
    return lay, x, rw, k


@pytest.mark.parametrize("fmt", [synth.FMT_ASYM_G64, synth.FMT_FP8_B128, synth.FMT_NVFP4])
@pytest.mark.parametrize("T", [4, 16])
def test_forward_det_bit_identical(fmt, T):
    lay, x, rw, k = _layer_case(fmt, T, seed=31 + T)
    say(f"[det] fmt={fmt} T={T}")
    ys = [_run(True, lay, x, rw, T, k) for _ in range(RUNS)]
    y0, idx0, _ = ys[0]
    for y, idx, _ in ys[1:]:
        assert torch.equal(idx, idx0)
        assert torch.equal(y.view(torch.int32), y0.view(torch.int32)), "runs differ"
    _, ir, gr, yr = oracle.moe_layer(lay, np_u16(x), T, k, router_w=np_u16(rw))
    assert np.array_equal(idx0.cpu().numpy(), ir)
    r, a = assert_close(y0.cpu().numpy(), yr, f"det fmt={fmt} T={T}")
    ya, _, _ = _run(False, lay, x, rw, T, k)
    d = (ya - y0).abs().max().item()
    say(f"[det] fmt={fmt} T={T}: rel L2 {r:.2e} max abs {a:.2e}; atomics vs slot order max diff {d:.2e}")
    assert d <= 1e-5 * max(1.0, y0.abs().max().item())


def test_forward_det_shared_and_residual():
    """Residual step bf16(x + y_prev) in the call, shared expert added after the slot-ordered sum."""
    T = 16
    lay, x, rw, k = _layer_case(synth.FMT_ASYM_G64, T, seed=7)
    sx = synth.random_shared(2048, 512, seed=7, device="cuda")
    yprev = synth.normal((T, 2048), 0.5, 7, "det/yprev", "cuda")
    outs = [_run(True, lay, x, rw, T, k, sx=sx, residual_y=yprev) for _ in range(RUNS)]
    y0, idx0, xo0 = outs[0]
    for y, idx, xo in outs[1:]:
        assert torch.equal(y.view(torch.int32), y0.view(torch.int32))
        assert torch.equal(xo, xo0)
    xin = oracle.residual(np_u16(x), yprev.cpu().numpy())
    assert np.array_equal(np_u16(xo0), xin)
    _, ir, gr, yr = oracle.moe_layer(lay, xin, T, k, router_w=np_u16(rw))
    yr = oracle.shared(sx.hidden, sx.inter, *[t.cpu().numpy() for t in sx.tensors()], xin, T, y_in=yr)
    assert np.array_equal(idx0.cpu().numpy(), ir)
    assert_close(y0.cpu().numpy(), yr, "det shared+residual")


def test_forward_det_chain_three_layers():
    """Three layers of the frame recipe chained through the library's own residual step (x_{l+1} =
    bf16(x_l + y_l) inside the next call), against the oracle's chain teacher-forced per layer: each
    layer's routing must match exactly on the inputs the library formed, and y must repeat bit for bit."""
    import quantized_moe_expert_amd as m
    case = synth.make_case(4, device="cuda", layers=3)
    T, k, H = case.T, case.k, case.H
    runs = []
    for _ in range(2):
        x, yprev, outs = case.x, None, []
        for l in range(3):
            lay, rw = case.layers[l], case.router_ws[l]
            y, idx, xo = _run(True, lay, x, rw, T, k, residual_y=yprev)
            xl = xo if xo is not None else x
            outs.append((y.clone(), idx.clone(), xl.clone()))
            x, yprev = xl, y
        runs.append(outs)
    for l in range(3):
        y, idx, xl = runs[0][l]
        y2, idx2, xl2 = runs[1][l]
        assert torch.equal(y.view(torch.int32), y2.view(torch.int32)), f"layer {l} differs between runs"
        x_np = np_u16(xl)
        if l > 0:  # the residual the library formed is the oracle's bf16(x + y) of its own previous layer
            yp, _, xp = runs[0][l - 1]
            assert np.array_equal(x_np, oracle.residual(np_u16(xp), yp.cpu().numpy()))
        _, ir, gr, yr = oracle.moe_layer(case.layers[l], x_np, T, k, router_w=np_u16(case.router_ws[l]))
        assert np.array_equal(idx.cpu().numpy(), ir)
        r, a = assert_close(y.cpu().numpy(), yr, f"det chain layer {l}")
        say(f"[det chain] layer {l}: rel L2 {r:.2e} max abs {a:.2e}")
    del m
