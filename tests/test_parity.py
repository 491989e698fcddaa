"""HIP path against the CPU oracle, through the C ABI (needs an MI355X).

Bars: dequantised weights, router logits, expert indices, histogram, offsets
and permutation bit-exact; gates within 1e-6 relative; layer outputs within
relative L2 2e-3 and max abs 1e-2 of the fp64 oracle.  Inputs are the seeded
synthetic workloads (synth.make_case) at full size, plus small and ragged
shapes; every token of the full-size layers is compared.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import (GATE_RTOL, assert_close, hip_experts, hip_route, np_u16, oracle_route, oracle_y)

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


def get_case(cfg, **kw):
    key = (cfg, tuple(sorted(kw.items())))
    if key not in _cases:
        say(f"[gen] config {cfg} {kw}")
        _cases[key] = synth.make_case(cfg, device="cuda", **kw)
        torch.cuda.synchronize()
    return _cases[key]


# ------------------------------------------------------------------ dequant

@pytest.mark.parametrize("fmt", [synth.FMT_ASYM_G64, synth.FMT_SYM_G128])
@pytest.mark.parametrize("shape", [(3, 256, 128), (2, 2048, 512)])
def test_dequant_bit_exact(fmt, shape):
    import quantized_moe_expert_amd as m
    E, H, I = shape
    say(f"[dequant] fmt={fmt} E={E} H={H} I={I}")
    lay = synth.random_layer(E, H, I, fmt, seed=5, device="cuda")
    host = oracle.layer_np(lay)
    g = synth.GROUP[fmt]
    for e in range(E):
        for proj in range(3):
            N, K = (H, I) if proj == 2 else (I, H)
            out = torch.empty((N, K), dtype=torch.float32, device="cuda")
            m.moe_q4_dequant(lay, e, proj, out)
            ref = oracle.dequant(fmt, host[proj][e], host[3 + proj][e], N, K)
            got = out.cpu().numpy()
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (e, proj)
    del g


def test_dequant_generated_layer_bit_exact():
    import quantized_moe_expert_amd as m
    case = get_case(1)
    lay = case.layers[0]
    host = oracle.layer_np(lay)
    for e in (0, 7, 15):
        out = torch.empty((lay.inter, lay.hidden), dtype=torch.float32, device="cuda")
        m.moe_q4_dequant(lay, e, 1, out)
        ref = oracle.dequant(lay.fmt, host[1][e], host[4][e], lay.inter, lay.hidden)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# -------------------------------------------------------------------- route

def _check_route(lg_gpu, idx_gpu, gate_gpu, lg_ref, idx_ref, gate_ref, compare_logits=True):
    if compare_logits:
        got = np_u16(lg_gpu)
        assert np.array_equal(got, lg_ref), f"{int((got != lg_ref).sum())} logits differ"
    assert np.array_equal(idx_gpu.cpu().numpy(), idx_ref), "expert indices differ"
    g = gate_gpu.cpu().numpy().astype(np.float64)
    assert np.allclose(g, gate_ref, rtol=GATE_RTOL, atol=0), float(np.max(np.abs(g / gate_ref - 1)))


@pytest.mark.parametrize("cfg", [1, 2])
def test_route_configs(cfg):
    case = get_case(cfg)
    say(f"[route] config {cfg}")
    lg, idx, gate = hip_route(case.x, case.router_w, None, case.T, case.H, case.E, case.k)
    lr, ir, gr = oracle_route(case, np_u16(case.x))
    _check_route(lg, idx, gate, lr, ir, gr)


@pytest.mark.parametrize("T,H,E,k", [(64, 2048, 256, 8), (300, 256, 16, 2), (5, 512, 1000, 32), (3, 64, 8, 8)])
def test_route_gemv_shapes(T, H, E, k):
    say(f"[route] T={T} H={H} E={E} k={k}")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 1, "rt/x", "cuda"))
    wr = synth.bf16_bits(synth.normal((E, H), 0.05, 1, "rt/w", "cuda"))
    bias = synth.normal((E,), 0.3, 1, "rt/b", "cuda")
    for b in (None, bias):
        lg, idx, gate = hip_route(x, wr, None, T, H, E, k, bias=b)
        lr = oracle.router(np_u16(x), np_u16(wr), T, H, E, None if b is None else b.cpu().numpy())
        ir, gr = oracle.topk(lr, T, E, k)
        _check_route(lg, idx, gate, lr, ir, gr)


@pytest.mark.parametrize("T,E,k", [(300, 256, 8), (50, 16, 2), (7, 9, 9), (4096, 256, 8)])
def test_route_given_logits_with_ties(T, E, k):
    """Logits from a handful of values: ties at the k-th place are everywhere."""
    say(f"[route ties] T={T} E={E} k={k}")
    g = synth.generator(3, "ties", "cuda")
    vals = torch.randint(-3, 4, (T, E), generator=g, device="cuda").float() * 0.25
    lg_in = synth.bf16_bits(vals)
    lg, idx, gate = hip_route(None, None, lg_in, T, 0, E, k)
    lr = np_u16(lg_in)
    ir, gr = oracle.topk(lr, T, E, k)
    _check_route(lg, idx, gate, lr, ir, gr)


def test_route_all_equal_and_zipf():
    T, E, k = 8, 256, 8
    lg_in = synth.bf16_bits(torch.full((T, E), 0.5, device="cuda"))
    _, idx, gate = hip_route(None, None, lg_in, T, 0, E, k)
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(k), (T, 1)))
    assert np.all(gate.cpu().numpy() == np.float32(1.0 / k))
    case = get_case(3)
    lg, idx, gate = hip_route(None, None, case.logits, case.T, case.H, case.E, case.k)
    lr, ir, gr = oracle_route(case, np_u16(case.x))
    _check_route(lg, idx, gate, lr, ir, gr, compare_logits=False)


# -------------------------------------------------------------------- group

def _hip_group(idx, T, k, E):
    import quantized_moe_expert_amd as m
    ws = torch.empty(max(m.workspace_size(m.WS_GROUP, T, E, k, 64, 64), 256), dtype=torch.uint8, device="cuda")
    cnt = torch.empty(E, dtype=torch.int32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    m.moe_q4_group(idx, T, k, E, cnt, off, perm, inv, ws)
    return [t.cpu().numpy() for t in (cnt, off, perm, inv)]


@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (4, 2, 16), (16, 8, 256), (32, 8, 256), (64, 4, 16), (64, 8, 256),
                                   (128, 8, 256), (129, 8, 256), (512, 8, 256), (4096, 8, 256), (333, 3, 1000)])
def test_group_exact(T, k, E):
    say(f"[group] T={T} k={k} E={E}")
    g = synth.generator(4, f"grp/{T}/{k}/{E}", "cuda")
    idx = torch.argsort(torch.rand((T, E), generator=g, device="cuda"), dim=1)[:, :k].to(torch.int32).contiguous()
    got = _hip_group(idx, T, k, E)
    ref = oracle.group(idx.cpu().numpy(), T, k, E)
    for name, a, b in zip(("cnt", "off", "perm", "inv"), got, ref):
        assert np.array_equal(a, b), name


def test_group_zipf_skew():
    case = get_case(3)
    _, idx, _ = hip_route(None, None, case.logits, case.T, case.H, case.E, case.k)
    got = _hip_group(idx, case.T, case.k, case.E)
    ref = oracle.group(idx.cpu().numpy(), case.T, case.k, case.E)
    for name, a, b in zip(("cnt", "off", "perm", "inv"), got, ref):
        assert np.array_equal(a, b), name
    say(f"[zipf] active experts {int((ref[0] > 0).sum())}, max load {int(ref[0].max())}, "
        f"median {int(np.median(ref[0]))}")


# -------------------------------------------------------------------- layer

def _layer_parity(case, mode, tokens=None, layer=0):
    lay = case.layers[layer]
    x_np = np_u16(case.x)
    rw = case.router_ws[layer] if case.router_ws else None
    lg, idx, gate = hip_route(case.x if rw is not None else None, rw, case.logits, case.T, case.H, case.E, case.k)
    sub = np.arange(case.T) if tokens is None else np.asarray(tokens)
    if rw is not None:
        lr = oracle.router(np.ascontiguousarray(x_np[sub]), np_u16(rw), len(sub), case.H, case.E)
    else:
        lr = np.ascontiguousarray(np_u16(case.logits)[sub])
    ir, gr = oracle.topk(lr, len(sub), case.E, case.k)
    assert np.array_equal(idx.cpu().numpy()[sub], ir), "expert indices differ"
    y = hip_experts(mode, lay, case.x, idx, gate, case.k)
    torch.cuda.synchronize()
    yr = oracle_y(lay, x_np, ir, gr, case.k, tokens=sub)
    r, a = assert_close(y.cpu().numpy()[sub], yr, f"{case.name} {mode}")
    say(f"[{mode}] {case.name} T={case.T}: rel L2 {r:.2e}, max abs {a:.2e}")
    return y


@pytest.mark.parametrize("cfg", [1, 2])
def test_decode_configs(cfg):
    _layer_parity(get_case(cfg), "decode")


def test_decode_frame_layer():
    """One layer of the 16-token frame recipe (RTN weights, GEMV router)."""
    _layer_parity(get_case(4, layers=1), "decode")


@pytest.mark.parametrize("cfg", [1, 3])
def test_prefill_configs(cfg):
    _layer_parity(get_case(cfg), "prefill")


def test_prefill_long_sym_all_tokens():
    """The 4096-token symmetric-g128 layer: every token against the oracle."""
    _layer_parity(get_case(5), "prefill")


def test_forward_long_sym_packed_all_tokens():
    """The long-prompt layer as the benchmark runs it: moe_q4_forward with
    the logits given and the prefill copy of the weights (top-k, grouping
    count and x conversion in one launch, then the grouped GEMMs); every
    token against the oracle."""
    import quantized_moe_expert_amd as m
    case = get_case(5)
    lay = case.layers[0]
    pk = m.prefill_pack(lay)
    st = m.layer_struct(lay, pack=pk)
    lg, idx, gate, y, _, _ = _forward(st, case.x, None, case.logits, case.T, case.k)
    torch.cuda.synchronize()
    ir, gr = oracle.topk(np_u16(case.logits), case.T, case.E, case.k)
    assert np.array_equal(idx.cpu().numpy(), ir)
    r, a = assert_close(y.cpu().numpy(), oracle_y(lay, np_u16(case.x), ir, gr, case.k), "forward long packed")
    say(f"[forward packed] config 5, all 4096 tokens: rel L2 {r:.2e}, max abs {a:.2e}")


@pytest.mark.parametrize("mode", ["decode", "prefill"])
@pytest.mark.parametrize("fmt", [synth.FMT_ASYM_G64, synth.FMT_SYM_G128])
@pytest.mark.parametrize("T", [1, 37, 200])
def test_layer_ragged(mode, fmt, T):
    """Ragged token counts on a 64-expert layer with random codes and scales."""
    H, I, E, k = 512, 256, 64, 6
    say(f"[ragged] {mode} fmt={fmt} T={T}")
    lay = synth.random_layer(E, H, I, fmt, seed=9, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 9, f"rg/x/{T}", "cuda"))
    wr = synth.bf16_bits(synth.normal((E, H), 0.05, 9, "rg/w", "cuda"))
    lg, idx, gate = hip_route(x, wr, None, T, H, E, k)
    lr = oracle.router(np_u16(x), np_u16(wr), T, H, E)
    ir, gr = oracle.topk(lr, T, E, k)
    assert np.array_equal(idx.cpu().numpy(), ir)
    y = hip_experts(mode, lay, x, idx, gate, k)
    yr = oracle.experts(fmt, E, H, I, *oracle.layer_np(lay), np_u16(x), ir, gr, T, k)
    assert_close(y.cpu().numpy(), yr, f"ragged {mode}")


@pytest.mark.parametrize("T", [1, 2, 3, 5, 7])
def test_decode_last_experts(T):
    """Tokens routed to the highest-numbered experts, at token counts whose
    row chunking does not divide the projections evenly: every weight row the
    kernels touch must lie inside the layer (regression: a chunk past the last
    row of the last expert read beyond the weights)."""
    H, I, E, k = 2048, 512, 256, 8
    say(f"[last experts] T={T}")
    lay = synth.random_layer(E, H, I, synth.FMT_ASYM_G64, seed=11, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 11, f"le/x/{T}", "cuda"))
    lg = np.zeros((T, E), dtype=np.float32)
    for t in range(T):
        lg[t, E - k - t % 3:] = np.linspace(1.0, 2.0, k + t % 3)  # top-k inside the last k + 2 experts
    lg_bits = synth.bf16_bits(torch.from_numpy(lg).to("cuda"))
    _, idx, gate = hip_route(None, None, lg_bits, T, H, E, k)
    ir, gr = oracle.topk(np_u16(lg_bits), T, E, k)
    assert np.array_equal(idx.cpu().numpy(), ir)
    assert int(idx.max()) == E - 1
    yr = oracle.experts(synth.FMT_ASYM_G64, E, H, I, *oracle.layer_np(lay), np_u16(x), ir, gr, T, k)
    for mode in ("decode", "prefill"):
        y = hip_experts(mode, lay, x, idx, gate, k)
        assert_close(y.cpu().numpy(), yr, f"last experts {mode} T={T}")


def test_decode_and_prefill_agree():
    case = get_case(4, layers=1, T=64)
    lay = case.layers[0]
    _, idx, gate = hip_route(case.x, case.router_ws[0], None, case.T, case.H, case.E, case.k)
    yd = hip_experts("decode", lay, case.x, idx, gate, case.k).cpu().numpy()
    yp = hip_experts("prefill", lay, case.x, idx, gate, case.k).cpu().numpy()
    assert_close(yp, yd, "prefill vs decode")


def test_decode_repeatable():
    """Float atomics may add the k slot outputs of a token in any order: runs
    agree to rounding, not bit for bit."""
    case = get_case(4, layers=1)
    lay = case.layers[0]
    _, idx, gate = hip_route(case.x, case.router_ws[0], None, case.T, case.H, case.E, case.k)
    y1 = hip_experts("decode", lay, case.x, idx, gate, case.k).cpu().numpy().astype(np.float64)
    y2 = hip_experts("decode", lay, case.x, idx, gate, case.k).cpu().numpy().astype(np.float64)
    assert np.linalg.norm(y1 - y2) <= 1e-6 * np.linalg.norm(y1)


def test_residual_bit_exact():
    import quantized_moe_expert_amd as m
    n = 16 * 2048 + 5
    x = synth.bf16_bits(synth.normal((n,), 1.0, 2, "res/x", "cuda"))
    y = synth.normal((n,), 0.7, 2, "res/y", "cuda")
    out = torch.empty_like(x)
    m.moe_q4_residual_bf16(x, y, n, out)
    ref = oracle.residual(np_u16(x), y.cpu().numpy())
    assert np.array_equal(np_u16(out), ref)


def test_frame_chain_layers():
    """Frame recipe (16 tokens, RTN g64, own router per layer), 3 layers: each
    layer runs on the oracle's own chain input x_l (teacher-forced), so a
    near-tie flip upstream cannot hide a downstream error."""
    case = get_case(4, layers=3)
    x_np = np_u16(case.x)
    for l in range(3):
        lay, rw = case.layers[l], case.router_ws[l]
        xl = torch.from_numpy(x_np.view(np.int16).copy()).cuda()
        lg, idx, gate = hip_route(xl, rw, None, case.T, case.H, case.E, case.k)
        lr = oracle.router(x_np, np_u16(rw), case.T, case.H, case.E)
        ir, gr = oracle.topk(lr, case.T, case.E, case.k)
        assert np.array_equal(np_u16(lg), lr)
        assert np.array_equal(idx.cpu().numpy(), ir)
        y = hip_experts("decode", lay, xl, idx, gate, case.k)
        yr = oracle_y(lay, x_np, ir, gr, case.k)
        r, a = assert_close(y.cpu().numpy(), yr, f"frame layer {l}")
        say(f"[frame] layer {l}: rel L2 {r:.2e} max abs {a:.2e}")
        x_np = oracle.residual(x_np, yr)


# ------------------------------------------------------------ fused forward

def _forward(lay, x, rw, logits, T, k, residual_y=None, ws=None):
    import quantized_moe_expert_amd as m
    E, H = lay.num_experts, lay.hidden
    if ws is None:
        ws = torch.zeros(max(m.workspace_size(m.WS_FORWARD, T, E, k, H, lay.inter), 256), dtype=torch.uint8,
                         device="cuda")
        m.moe_q4_workspace_init(ws)
    lg = logits.clone() if logits is not None else torch.empty((T, E), dtype=torch.int16, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    xo = torch.empty_like(x) if residual_y is not None else None
    m.moe_q4_forward(x, residual_y, xo, rw, None, lg, T, k, lay, idx, gate, y, ws)
    return lg, idx, gate, y, xo, ws


@pytest.mark.parametrize("cfg,T", [(2, None), (4, None), (3, 128)])
def test_forward_timed_matches_forward(cfg, T):
    """The timed entry point runs the same kernels (both decode routing
    variants and the prefill path) and records positive kernel spans."""
    import quantized_moe_expert_amd as m
    case = get_case(cfg, layers=1, T=T) if cfg == 4 else (get_case(cfg, T=T) if T else get_case(cfg))
    lay = case.layers[0]
    rw = case.router_ws[0] if case.router_ws else None
    say(f"[forward timed] cfg={cfg} T={case.T}")
    lg, idx, gate, y, _, ws = _forward(lay, case.x, rw, case.logits, case.T, case.k)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    lg2 = case.logits.clone() if case.logits is not None else torch.empty_like(lg)
    idx2, gate2 = torch.empty_like(idx), torch.empty_like(gate)
    y2 = torch.full_like(y, float("nan"))
    m.moe_q4_forward_timed(case.x, None, None, rw, None, lg2, case.T, case.k, lay, idx2, gate2, y2, ws,
                           [e.cuda_event for e in evs])
    torch.cuda.synchronize()
    assert torch.equal(lg, lg2) and torch.equal(idx, idx2) and torch.equal(gate, gate2)
    assert_close(y2.cpu().numpy(), y.cpu().numpy(), "timed vs plain forward")
    assert evs[0].elapsed_time(evs[1]) > 0 and evs[2].elapsed_time(evs[3]) > 0


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_forward_decode_configs(cfg):
    case = get_case(cfg, layers=1) if cfg == 4 else get_case(cfg)
    lay, rw = case.layers[0], case.router_ws[0]
    x_np = np_u16(case.x)
    ws = None
    for rep in range(2):  # the second call reuses the workspace (counter left at zero)
        lg, idx, gate, y, _, ws = _forward(lay, case.x, rw, None, case.T, case.k, ws=ws)
        lr = oracle.router(x_np, np_u16(rw), case.T, case.H, case.E)
        ir, gr = oracle.topk(lr, case.T, case.E, case.k)
        _check_route(lg, idx, gate, lr, ir, gr)
        r, a = assert_close(y.cpu().numpy(), oracle_y(lay, x_np, ir, gr, case.k), f"forward cfg {cfg}")
        say(f"[forward] config {cfg} call {rep}: rel L2 {r:.2e} max abs {a:.2e}")


def test_forward_given_logits_and_prefill_path():
    case = get_case(3)
    lay = case.layers[0]
    x_np = np_u16(case.x)
    for T in (16, 200):  # decode path, then prefill path
        lg, idx, gate, y, _, _ = _forward(lay, case.x[:T].contiguous(), None, case.logits[:T].contiguous(), T,
                                          case.k)
        lr = np.ascontiguousarray(np_u16(case.logits)[:T])
        ir, gr = oracle.topk(lr, T, case.E, case.k)
        assert np.array_equal(idx.cpu().numpy(), ir)
        assert_close(y.cpu().numpy(), oracle_y(lay, np.ascontiguousarray(x_np[:T]), ir, gr, case.k),
                     f"forward T={T}")


@pytest.mark.parametrize("fmt", [synth.FMT_ASYM_G64, synth.FMT_SYM_G128, synth.FMT_FP8_B128, synth.FMT_NVFP4])
@pytest.mark.parametrize("T,k", [(300, 8), (229, 6), (1100, 1), (40, 32), (401, 3)])
def test_forward_prefill_prep(fmt, T, k):
    """moe_q4_forward above 1024 (token, slot) pairs takes the top-k, the
    grouping's count and the f16 rows of x in one launch per 64-pair chunk:
    k = 6 and 3 put tokens across chunk boundaries, every T here leaves a
    partial last chunk, k = 1 gives 64 tokens per chunk and k = 32 two.  Expert indices bit-exact,
    gates and outputs against the oracle, for every weight format."""
    H, I, E = 512, 256, 64
    say(f"[prep] fmt={fmt} T={T} k={k}")
    lay = synth.random_layer(E, H, I, fmt, seed=13, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 13, f"prep/x/{T}", "cuda"))
    logits = synth.bf16_bits(synth.normal((T, E), 1.0, 13, f"prep/l/{T}", "cuda"))
    lg, idx, gate, y, _, _ = _forward(lay, x, None, logits, T, k)
    ir, gr = oracle.topk(np_u16(logits), T, E, k)
    assert np.array_equal(idx.cpu().numpy(), ir), "expert indices differ"
    assert np.allclose(gate.cpu().numpy(), gr, rtol=GATE_RTOL, atol=0), "gates differ"
    assert_close(y.cpu().numpy(), oracle_y(lay, np_u16(x), ir, gr, k), f"prep fmt={fmt} T={T} k={k}")


def test_forward_residual_chain():
    """Frame recipe, 3 layers through moe_q4_forward with the residual fused:
    layer l gets the oracle's x_{l-1} and y_{l-1}; its x_l must equal the
    oracle's bit for bit, then routing and y as usual."""
    case = get_case(4, layers=3)
    x_prev = np_u16(case.x)
    y_prev = None
    for l in range(3):
        lay, rw = case.layers[l], case.router_ws[l]
        xg = torch.from_numpy(x_prev.view(np.int16).copy()).cuda()
        yg = torch.from_numpy(y_prev.copy()).cuda() if y_prev is not None else None
        lg, idx, gate, y, xo, _ = _forward(lay, xg, rw, None, case.T, case.k, residual_y=yg)
        x_l = oracle.residual(x_prev, y_prev) if y_prev is not None else x_prev
        if xo is not None:
            assert np.array_equal(np_u16(xo), x_l), "residual input differs"
        lr = oracle.router(x_l, np_u16(rw), case.T, case.H, case.E)
        ir, gr = oracle.topk(lr, case.T, case.E, case.k)
        _check_route(lg, idx, gate, lr, ir, gr)
        yr = oracle_y(lay, x_l, ir, gr, case.k)
        r, a = assert_close(y.cpu().numpy(), yr, f"chain layer {l}")
        say(f"[chain] layer {l}: rel L2 {r:.2e} max abs {a:.2e}")
        x_prev, y_prev = x_l, yr


@pytest.mark.parametrize("T,E,k", [(60, 300, 6), (3, 1000, 32)])
def test_forward_wide_router(T, E, k):
    """Decode-size forward where T x E exceeds the one-launch routing's LDS
    (separate router, top-k and grouping launches) or uses many experts."""
    H, I = 512, 256
    say(f"[forward wide] T={T} E={E} k={k}")
    lay = synth.random_layer(E, H, I, synth.FMT_ASYM_G64, seed=11, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 11, f"fw/x/{T}", "cuda"))
    wr = synth.bf16_bits(synth.normal((E, H), 0.05, 11, f"fw/w/{E}", "cuda"))
    lg, idx, gate, y, _, _ = _forward(lay, x, wr, None, T, k)
    lr = oracle.router(np_u16(x), np_u16(wr), T, H, E)
    ir, gr = oracle.topk(lr, T, E, k)
    _check_route(lg, idx, gate, lr, ir, gr)
    yr = oracle.experts(lay.fmt, E, H, I, *oracle.layer_np(lay), np_u16(x), ir, gr, T, k)
    assert_close(y.cpu().numpy(), yr, f"forward wide T={T} E={E}")
