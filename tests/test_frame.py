"""moe_q4_frame against the oracle: a chain of MoE layers run as token lanes
on their own streams.

Each layer is checked from the input the GPU chain actually gave it: layer
j's input (x for j = 0, else the frame's x_chain[j - 1]) must equal the
oracle's residual step bf16(x_{j-1} + y_{j-1}) of the GPU's own previous
layer bit for bit; its logits (oracle router on that input) bit for bit, its
indices exactly, its gates to 1e-6, and its y to the output bar against the
oracle's experts on that input.  So a near-tie flip between the GPU's and the
oracle's chains cannot hide or fake an error.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import GATE_RTOL, assert_close, np_u16, oracle_y

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_expert_amd as m
    m.lib()  # fails loudly if the library was not built
    return torch.device("cuda")


_cases = {}
_streams = []


def lane_streams(n):
    """n streams at the default priority, made once and reused (a process
    gets only a few hardware queues)."""
    while len(_streams) < n:
        _streams.append(torch.cuda.Stream())
    return [torch.cuda.current_stream()] + _streams[:n - 1]


def frame_case(layers, T, fmt=None):
    key = (layers, T, fmt)
    if key not in _cases:
        say(f"[gen] frame recipe, {layers} layers, T={T}, format {fmt}")
        _cases[key] = synth.make_case(4, device="cuda", layers=layers, T=T, fmt=fmt)
        torch.cuda.synchronize()
    return _cases[key]


def run_frame(case, lanes, shared=None, events=None):
    import quantized_moe_expert_amd as m
    T, H, E, k, I = case.T, case.H, case.E, case.k, case.I
    n = len(case.layers)
    dev = "cuda"
    x_chain = torch.full((max(n - 1, 1), T, H), -1, dtype=torch.int16, device=dev)
    y_chain = torch.full((n, T, H), float("nan"), dtype=torch.float32, device=dev)
    lg = torch.empty((n, T, E), dtype=torch.int16, device=dev)
    idx = torch.full((n, T, k), -1, dtype=torch.int32, device=dev)
    gate = torch.empty((n, T, k), dtype=torch.float32, device=dev)
    sinter = shared[0].inter if shared else 0
    ws = torch.empty(max(m.frame_workspace_size(T, E, k, H, I, sinter, lanes), 256), dtype=torch.uint8,
                     device=dev)
    streams = lane_streams(lanes)
    main = torch.cuda.current_stream()
    for s in streams[1:]:
        s.wait_stream(main)  # the inputs above are ready on every lane
    m.moe_q4_frame(case.x, T, k, case.layers, case.router_ws, shared, x_chain if n > 1 else None, y_chain, lg,
                   idx, gate, lanes, streams, ws, events=events)
    for s in streams[1:]:
        main.wait_stream(s)
    torch.cuda.synchronize()
    return x_chain, y_chain, lg, idx, gate


def check_chain(case, lanes, out, shared=None, what="frame"):
    x_chain, y_chain, lg, idx, gate = out
    T, H, E, k = case.T, case.H, case.E, case.k
    x_in = np_u16(case.x)
    for j, lay in enumerate(case.layers):
        if j > 0:
            x_j = np_u16(x_chain[j - 1])
            expect = oracle.residual(x_in, y_chain[j - 1].cpu().numpy())
            assert np.array_equal(x_j, expect), f"{what} layer {j}: residual input differs"
            x_in = x_j
        lr = oracle.router(x_in, np_u16(case.router_ws[j]), T, H, E)
        ir, gr = oracle.topk(lr, T, E, k)
        assert np.array_equal(np_u16(lg[j]), lr), f"{what} layer {j}: logits differ"
        assert np.array_equal(idx[j].cpu().numpy(), ir), f"{what} layer {j}: expert indices differ"
        g = gate[j].cpu().numpy().astype(np.float64)
        assert np.allclose(g, gr, rtol=GATE_RTOL, atol=0), f"{what} layer {j}: gates"
        yr = oracle_y(lay, x_in, ir, gr, k)
        if shared is not None:
            sx = shared[j]
            yr = oracle.shared(sx.hidden, sx.inter, *[t.cpu().numpy() for t in sx.tensors()], x_in, T, y_in=yr)
        r, a = assert_close(y_chain[j].cpu().numpy(), yr, f"{what} layer {j}")
        say(f"[{what}] lanes {lanes} layer {j}: rel L2 {r:.2e} max abs {a:.2e}")


@pytest.mark.parametrize("lanes", [1, 2])
def test_frame_lanes_recipe(lanes):
    """The frame recipe (16 tokens, 256 experts, top-8, own router per
    layer), 3 layers, one lane and two lanes of 8 tokens (each lane routing
    in its expert launches)."""
    case = frame_case(3, 16)
    check_chain(case, lanes, run_frame(case, lanes))


@pytest.mark.parametrize("T,lanes", [(5, 2), (5, 3), (7, 4), (40, 2), (300, 2)])
def test_frame_lanes_ragged(T, lanes):
    """Uneven lanes (5 tokens as 2 + 3 and 1 + 2 + 2, 7 as 1 + 2 + 2 + 2),
    lanes of 20 tokens (160 pairs: the routing launch's one-block grouping
    instead of routing in the expert launches) and of 150 tokens (1200
    pairs: the prefill path, its grouped GEMMs side by side), 2 layers."""
    case = frame_case(2, T)
    check_chain(case, lanes, run_frame(case, lanes), what=f"frame T={T}")


@pytest.mark.parametrize("fmt", [synth.FMT_FP8_B128, synth.FMT_NVFP4])
def test_frame_lanes_formats(fmt):
    """Two lanes of 8 tokens, 2 layers, with block-FP8 and NVFP4 experts."""
    case = frame_case(2, 16, fmt)
    check_chain(case, 2, run_frame(case, 2), what=f"frame fmt {fmt}")


def test_frame_lanes_shared_expert():
    """Two lanes with each layer's shared expert (int8 sym g128) fused in the
    lanes' expert launches."""
    case = frame_case(2, 16)
    shared = [synth.make_shared(case.H, 512, 0, f"frame-test/L{j}/shared", device="cuda") for j in range(2)]
    torch.cuda.synchronize()
    check_chain(case, 2, run_frame(case, 2, shared=shared), shared=shared, what="frame+shared")


def test_frame_lanes_events():
    """With stage events, every lane's kernels record positive spans; the
    outputs are those of a run without events."""
    case = frame_case(2, 16)
    lanes = 2
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * lanes * 4)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    out = run_frame(case, lanes, events=[e.cuda_event for e in evs])
    check_chain(case, lanes, out, what="frame events")
    for i in range(0, len(evs), 4):
        assert evs[i].elapsed_time(evs[i + 1]) > 0
        assert evs[i + 2].elapsed_time(evs[i + 3]) > 0
