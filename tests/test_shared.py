"""Shared expert (int8 symmetric group 128) on the HIP path against the CPU
oracle, through the C ABI (needs an MI355X).

Bars: dequantised weights and expert indices bit-exact; outputs within the
layer tolerance (relative L2 2e-3, max abs 1e-2 against the fp64 oracle).
Inputs: the synthetic shared expert of the layer recipe (H = 2048, I = 512,
Gaussian weights encoded by synth.quantize_int8) at the decode, frame and
long prefill token counts (sampled tokens at 4096), plus random codes at the
smallest and largest supported shapes and ragged token counts; the layer
forward with a shared expert on each of its paths (routing inside the
expert launches, in the routing launch, shared items fused or on their own,
prefill).
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


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_expert_amd as m
    m.lib()
    return torch.device("cuda")


def host(sx):
    return [t.cpu().numpy() for t in sx.tensors()]


def hip_shared(sx, x, y=None, accumulate=False):
    import quantized_moe_expert_amd as m
    T = x.shape[0]
    ws = torch.empty(max(m.workspace_size(m.WS_SHARED, T, 1, 1, sx.hidden, sx.inter), 256), dtype=torch.uint8,
                     device="cuda")
    if y is None:
        y = torch.full((T, sx.hidden), float("nan"), dtype=torch.float32, device="cuda")
    m.moe_q4_shared(x, T, sx, y, accumulate, ws)
    return y


_shared = {}


def recipe_shared():
    if "recipe" not in _shared:
        _shared["recipe"] = synth.make_shared(2048, 512, seed=0, tag="layer_shared", device="cuda")
    return _shared["recipe"]


@pytest.mark.parametrize("shape", [(128, 128), (2048, 512), (512, 2048), (2048, 128)])
def test_dequant_int8_bit_exact(shape):
    import quantized_moe_expert_amd as m
    H, I = shape
    say(f"[dequant_int8] H={H} I={I}")
    sx = synth.random_shared(H, I, seed=3, device="cuda")
    hq = host(sx)
    for proj in range(3):
        N, K = (H, I) if proj == 2 else (I, H)
        out = torch.empty((N, K), dtype=torch.float32, device="cuda")
        m.moe_q4_dequant_int8(sx, proj, out)
        ref = oracle.dequant_int8(hq[proj], hq[3 + proj], N, K)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), proj


def test_dequant_int8_extreme_codes():
    """Codes -128, -127, 127 and zero, negative and subnormal scales decode exactly."""
    import quantized_moe_expert_amd as m
    H, I = 256, 128
    sx = synth.random_shared(H, I, seed=4, device="cuda")
    q = torch.tensor([-128, -127, 127, 0, 1, -1], dtype=torch.int8, device="cuda")
    sx.gate_q.view(-1).copy_(q.repeat(I * H // 6 + 1)[: I * H])
    s = torch.tensor([0x0001, 0x8400, 0x7bff, 0x0000, 0x3c00], dtype=torch.int32).to(torch.int16)
    sx.gate_s.view(-1).copy_(s.repeat(I * 2 // 5 + 1)[: I * 2].to("cuda"))
    out = torch.empty((I, H), dtype=torch.float32, device="cuda")
    m.moe_q4_dequant_int8(sx, 0, out)
    hq = host(sx)
    ref = oracle.dequant_int8(hq[0], hq[3], I, H)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("T", [1, 16, 64])
def test_shared_recipe(T):
    sx = recipe_shared()
    x = synth.bf16_bits(synth.normal((T, 2048), 1.0, 0, f"shared/x/{T}", "cuda"))
    say(f"[shared] recipe T={T}")
    y = hip_shared(sx, x)
    ref = oracle.shared(2048, 512, *host(sx), np_u16(x), T)
    r, a = assert_close(y.cpu().numpy(), ref, f"shared T={T}")
    say(f"[shared] T={T}: rel L2 {r:.2e}, max abs {a:.2e}")


def test_shared_long_prefill_sampled():
    sx = recipe_shared()
    T = 4096
    x = synth.bf16_bits(synth.normal((T, 2048), 1.0, 0, "shared/x/long", "cuda"))
    say(f"[shared] recipe T={T} (sampled)")
    y = hip_shared(sx, x).cpu().numpy()
    tokens = np.unique(np.concatenate([np.arange(0, T, 211), [1, T - 2, T - 1]]))
    ref = oracle.shared(2048, 512, *host(sx), np_u16(x), T, tokens=tokens)
    assert_close(y[tokens], ref, "shared long")


def test_shared_accumulate():
    """accumulate = 1 adds into the given y (the routed output of the layer)."""
    sx = recipe_shared()
    T = 7
    x = synth.bf16_bits(synth.normal((T, 2048), 1.0, 1, "shared/x/acc", "cuda"))
    y0 = synth.normal((T, 2048), 0.05, 1, "shared/y0", "cuda")
    y = hip_shared(sx, x, y=y0.clone(), accumulate=True)
    ref = oracle.shared(2048, 512, *host(sx), np_u16(x), T, y_in=y0.cpu().numpy())
    assert_close(y.cpu().numpy(), ref, "shared accumulate")


@pytest.mark.parametrize("shape", [(128, 128), (2048, 128), (128, 2048), (512, 256)])
@pytest.mark.parametrize("T", [1, 3, 37, 200])
def test_shared_ragged(shape, T):
    H, I = shape
    say(f"[shared] random H={H} I={I} T={T}")
    sx = synth.random_shared(H, I, seed=7, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 7, f"shared/rx/{H}/{T}", "cuda"))
    y = hip_shared(sx, x)
    ref = oracle.shared(H, I, *host(sx), np_u16(x), T)
    assert_close(y.cpu().numpy(), ref, f"shared {H}x{I} T={T}")


def test_shared_zero_tokens_is_a_no_op():
    import quantized_moe_expert_amd as m
    sx = recipe_shared()
    y = torch.full((1, 2048), 3.0, dtype=torch.float32, device="cuda")
    x = torch.zeros((1, 2048), dtype=torch.int16, device="cuda")
    m.moe_q4_shared(x, 0, sx, y, False, None)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())


# ------------------------------------------------------- layer with shared

def hip_forward_shared(lay, sx, x, k, router_w=None, logits=None, residual_y=None):
    import quantized_moe_expert_amd as m
    T, H, E = x.shape[0], lay.hidden, lay.num_experts
    nb = m.workspace_size(m.WS_FORWARD, T, E, k, H, lay.inter)
    if sx is not None:
        nb += m.workspace_size(m.WS_SHARED, T, 1, 1, H, sx.inter)
    ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device="cuda")
    m.moe_q4_workspace_init(ws)
    lg = torch.empty((T, E), dtype=torch.int16, device="cuda") if logits is None else logits.clone()
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    x_out = torch.empty_like(x) if residual_y is not None else None
    m.moe_q4_forward_ex(x, residual_y, x_out, router_w, None, lg, T, k, lay, sx, idx, gate, y, ws)
    torch.cuda.synchronize()
    return y, idx, x_out


def oracle_layer_shared(lay, sx, x_np, k, router_w=None, logits=None):
    T = x_np.shape[0]
    _, idx, gate, y = oracle.moe_layer(lay, x_np, T, k, router_w=None if router_w is None else np_u16(router_w),
                                       logits=None if logits is None else np_u16(logits))
    if sx is None:
        return idx, y
    return idx, oracle.shared(sx.hidden, sx.inter, *host(sx), x_np, T, y_in=y)


@pytest.mark.parametrize("T", [1, 16])
def test_forward_shared_recipe(T):
    """The frame layer recipe (E = 256, k = 8, GEMV router) with the synthetic
    shared expert: T = 1 routes inside the expert launches, T = 16 in the
    routing launch; both run the shared items inside the expert launches."""
    cfg = 2 if T == 1 else 4
    case = synth.make_case(cfg, device="cuda", layers=1) if cfg == 4 else synth.make_case(cfg, device="cuda")
    sx = recipe_shared()
    say(f"[forward+shared] {case.name} T={T}")
    y, idx, _ = hip_forward_shared(case.layers[0], sx, case.x, case.k, router_w=case.router_w)
    ir, yr = oracle_layer_shared(case.layers[0], sx, np_u16(case.x), case.k, router_w=case.router_w)
    assert np.array_equal(idx.cpu().numpy(), ir)
    r, a = assert_close(y.cpu().numpy(), yr, f"forward+shared T={T}")
    say(f"[forward+shared] T={T}: rel L2 {r:.2e}, max abs {a:.2e}")


@pytest.mark.parametrize("I_s", [256, 512])
@pytest.mark.parametrize("T", [1, 7, 37, 200])
def test_forward_shared_ragged(T, I_s):
    """E = 64 random layer (I = 256): I_s = 256 fuses the shared items into
    the decode launches, I_s = 512 runs them on their own; T = 200 takes the
    prefill path."""
    H, I, E, k = 512, 256, 64, 6
    say(f"[forward+shared] ragged T={T} I_s={I_s}")
    lay = synth.random_layer(E, H, I, synth.FMT_ASYM_G64, seed=11, device="cuda")
    sx = synth.random_shared(H, I_s, seed=11, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 11, f"fs/x/{T}", "cuda"))
    wr = synth.bf16_bits(synth.normal((E, H), 0.05, 11, "fs/w", "cuda"))
    y, idx, _ = hip_forward_shared(lay, sx, x, k, router_w=wr)
    ir, yr = oracle_layer_shared(lay, sx, np_u16(x), k, router_w=wr)
    assert np.array_equal(idx.cpu().numpy(), ir)
    assert_close(y.cpu().numpy(), yr, f"forward+shared ragged T={T} I_s={I_s}")


def test_forward_shared_residual_and_given_logits():
    """Residual input bf16(x + y_prev) and given logits, with the shared expert."""
    H, I, E, k, T = 512, 256, 64, 6, 9
    lay = synth.random_layer(E, H, I, synth.FMT_SYM_G128, seed=13, device="cuda")
    sx = synth.random_shared(H, I, seed=13, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 13, "fsr/x", "cuda"))
    yprev = synth.normal((T, H), 0.3, 13, "fsr/y", "cuda")
    lg = synth.bf16_bits(synth.normal((T, E), 1.0, 13, "fsr/lg", "cuda"))
    y, idx, x_out = hip_forward_shared(lay, sx, x, k, logits=lg, residual_y=yprev)
    xin = oracle.residual(np_u16(x), yprev.cpu().numpy())
    assert np.array_equal(np_u16(x_out), xin)
    ir, yr = oracle_layer_shared(lay, sx, xin, k, logits=lg)
    assert np.array_equal(idx.cpu().numpy(), ir)
    assert_close(y.cpu().numpy(), yr, "forward+shared residual")


def test_forward_without_shared_unchanged():
    """forward_ex with no shared expert equals moe_q4_forward bit for bit."""
    import quantized_moe_expert_amd as m
    case = synth.make_case(4, device="cuda", layers=1)
    lay, T, k = case.layers[0], case.T, case.k
    y1, _, _ = hip_forward_shared(lay, None, case.x, k, router_w=case.router_w)
    ws = torch.zeros(m.workspace_size(m.WS_FORWARD, T, case.E, k, case.H, case.I), dtype=torch.uint8, device="cuda")
    m.moe_q4_workspace_init(ws)
    lg = torch.empty((T, case.E), dtype=torch.int16, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y2 = torch.empty((T, case.H), dtype=torch.float32, device="cuda")
    m.moe_q4_forward(case.x, None, None, case.router_w, None, lg, T, k, lay, idx, gate, y2, ws)
    ir, yr = oracle_layer_shared(lay, None, np_u16(case.x), k, router_w=case.router_w)
    assert_close(y1.cpu().numpy(), yr, "forward_ex without shared")
    assert_close(y2.cpu().numpy(), yr, "forward")


@pytest.mark.parametrize("T", [64, 65, 300])
def test_shared_gemv_gemm_threshold(T):
    """64 tokens take the GEMVs, 65 and more the matrix-core GEMMs (a ragged
    last tile at 65 and 300); both against the oracle, with accumulate."""
    sx = recipe_shared()
    x = synth.bf16_bits(synth.normal((T, 2048), 1.0, 2, f"shared/thr/{T}", "cuda"))
    y0 = synth.normal((T, 2048), 0.05, 2, f"shared/thr/y/{T}", "cuda")
    y = hip_shared(sx, x, y=y0.clone(), accumulate=True)
    ref = oracle.shared(2048, 512, *host(sx), np_u16(x), T, y_in=y0.cpu().numpy())
    r, a = assert_close(y.cpu().numpy(), ref, f"shared threshold T={T}")
    say(f"[shared] T={T} accumulate: rel L2 {r:.2e}, max abs {a:.2e}")
