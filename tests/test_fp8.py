"""Block-FP8 routed experts (E4M3 codes, one float32 scale per 128 x 128
block) on the HIP path against the CPU oracle, through the C ABI (needs an
MI355X).

Bars: dequantised weights and expert indices bit-exact; layer outputs within
relative L2 2e-3 and max abs 1e-2 of the fp64 oracle.  Inputs: the layer
recipe (H = 2048, 256 experts, top-8, I = 512) with N(0, 0.02) weights
encoded per 128 x 128 block (synth.quantize_fp8), at 1 and 16 tokens
(decode GEMVs) and at 512 (Zipf popularity) and 4096 tokens (grouped GEMMs,
every token), and random codes (subnormals included) at small, ragged
and extreme shapes, with all-zero blocks.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import assert_close, hip_route, np_u16

pytestmark = pytest.mark.gpu
FP8 = synth.FMT_FP8_B128


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_expert_amd as m
    m.lib()
    return torch.device("cuda")


@pytest.mark.parametrize("shape", [(2, 256, 128), (2, 2048, 512), (1, 128, 2048)])
def test_dequant_fp8_bit_exact(shape):
    import quantized_moe_expert_amd as m
    E, H, I = shape
    say(f"[dequant fp8] E={E} H={H} I={I}")
    lay = synth.random_layer(E, H, I, FP8, seed=5, device="cuda")
    host = oracle.layer_np(lay)
    for e in range(E):
        for proj in range(3):
            N, K = (H, I) if proj == 2 else (I, H)
            out = torch.empty((N, K), dtype=torch.float32, device="cuda")
            m.moe_q4_dequant(lay, e, proj, out)
            ref = oracle.dequant(FP8, host[proj][e], host[3 + proj][e], N, K)
            assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), (e, proj)


def test_dequant_fp8_every_code():
    """All 254 finite codes (and both zeros) in one matrix, with negative and tiny block scales."""
    import quantized_moe_expert_amd as m
    H, I = 256, 128
    lay = synth.random_layer(1, H, I, FP8, seed=6, device="cuda")
    codes = torch.tensor([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=torch.uint8)
    lay.gate_q.view(-1).copy_(codes.repeat(I * H // len(codes) + 1)[: I * H].to("cuda"))
    lay.gate_sm.view(-1).copy_(torch.tensor([-3.0e-4, 1.0, 2.0 ** -20, 448.0], dtype=torch.float32, device="cuda")[:2])
    out = torch.empty((I, H), dtype=torch.float32, device="cuda")
    m.moe_q4_dequant(lay, 0, 0, out)
    host = oracle.layer_np(lay)
    ref = oracle.dequant(FP8, host[0][0], host[3][0], I, H)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


_layers = {}


def recipe_layer():
    if "r" not in _layers:
        say("[gen] fp8 recipe layer")
        _layers["r"] = synth.make_layer(256, 2048, 512, FP8, seed=0, tag="fp8_layer", device="cuda")
        _layers["w"] = synth.bf16_bits(synth.normal((256, 2048), 0.02, 0, "fp8_layer/router", "cuda"))
    return _layers["r"], _layers["w"]


def hip_forward(lay, x, k, router_w=None, logits=None, residual_y=None):
    import quantized_moe_expert_amd as m
    T, H, E = x.shape[0], lay.hidden, lay.num_experts
    ws = torch.zeros(max(m.workspace_size(m.WS_FORWARD, T, E, k, H, lay.inter), 256), dtype=torch.uint8,
                     device="cuda")
    m.moe_q4_workspace_init(ws)
    lg = torch.empty((T, E), dtype=torch.int16, device="cuda") if logits is None else logits.clone()
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    x_out = torch.empty_like(x) if residual_y is not None else None
    m.moe_q4_forward(x, residual_y, x_out, router_w, None, lg, T, k, lay, idx, gate, y, ws)
    torch.cuda.synchronize()
    return y, idx


@pytest.mark.parametrize("T", [1, 16])
def test_fp8_forward_recipe(T):
    lay, wr = recipe_layer()
    x = synth.bf16_bits(synth.normal((T, 2048), 1.0, 0, f"fp8/x/{T}", "cuda"))
    say(f"[fp8 forward] recipe T={T}")
    y, idx = hip_forward(lay, x, 8, router_w=wr)
    _, ir, _, yr = oracle.moe_layer(lay, np_u16(x), T, 8, router_w=np_u16(wr))
    assert np.array_equal(idx.cpu().numpy(), ir)
    r, a = assert_close(y.cpu().numpy(), yr, f"fp8 forward T={T}")
    say(f"[fp8 forward] T={T}: rel L2 {r:.2e}, max abs {a:.2e}")


def test_fp8_forward_many_tokens_sampled():
    """512 tokens: the forward call runs the GEMV kernels after separate routing launches."""
    lay, wr = recipe_layer()
    T = 512
    x = synth.bf16_bits(synth.normal((T, 2048), 1.0, 0, "fp8/x/many", "cuda"))
    y, idx = hip_forward(lay, x, 8, router_w=wr)
    tokens = np.array([0, 1, 77, 255, 256, 400, 510, 511])
    _, ir, _, yr = oracle.moe_layer(lay, np_u16(x), T, 8, router_w=np_u16(wr), tokens=tokens)
    assert np.array_equal(idx.cpu().numpy()[tokens], ir)
    r, a = assert_close(y.cpu().numpy()[tokens], yr, "fp8 forward T=512")
    say(f"[fp8 forward] T=512 sampled: rel L2 {r:.2e}, max abs {a:.2e}")


@pytest.mark.parametrize("T", [1, 37, 200])
def test_fp8_decode_ragged(T):
    """Random codes on a 64-expert layer (H = 512, I = 256) through moe_q4_decode."""
    import quantized_moe_expert_amd as m
    H, I, E, k = 512, 256, 64, 6
    lay = synth.random_layer(E, H, I, FP8, seed=9, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 9, f"fp8/rx/{T}", "cuda"))
    wr = synth.bf16_bits(synth.normal((E, H), 0.05, 9, "fp8/rw", "cuda"))
    lg, idx, gate = hip_route(x, wr, None, T, H, E, k)
    ws = torch.empty(m.workspace_size(m.WS_DECODE, T, E, k, H, I), dtype=torch.uint8, device="cuda")
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    m.moe_q4_decode(x, idx, gate, T, k, lay, y, ws)
    lr = oracle.router(np_u16(x), np_u16(wr), T, H, E)
    ir, gr = oracle.topk(lr, T, E, k)
    assert np.array_equal(idx.cpu().numpy(), ir)
    yr = oracle.experts(FP8, E, H, I, *oracle.layer_np(lay), np_u16(x), ir, gr, T, k)
    assert_close(y.cpu().numpy(), yr, f"fp8 decode T={T}")


@pytest.mark.parametrize("shape", [(128, 2048), (2048, 128)])
def test_fp8_extreme_shapes(shape):
    H, I = shape
    E, k, T = 8, 2, 5
    lay = synth.random_layer(E, H, I, FP8, seed=12, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 12, f"fp8/ex/{H}", "cuda"))
    lg = synth.bf16_bits(synth.normal((T, E), 1.0, 12, f"fp8/exl/{H}", "cuda"))
    y, idx = hip_forward(lay, x, k, logits=lg)
    _, ir, _, yr = oracle.moe_layer(lay, np_u16(x), T, k, logits=np_u16(lg))
    assert np.array_equal(idx.cpu().numpy(), ir)
    assert_close(y.cpu().numpy(), yr, f"fp8 {H}x{I}")


def test_fp8_forward_with_shared_and_residual():
    """A frame-like layer step: residual input, GEMV router, FP8 experts and the int8 shared expert."""
    import quantized_moe_expert_amd as m
    lay, wr = recipe_layer()
    T, k, H = 16, 8, 2048
    sx = synth.make_shared(H, 512, seed=0, tag="fp8_layer_shared", device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 3, "fp8/x/res", "cuda"))
    yprev = synth.normal((T, H), 0.2, 3, "fp8/yprev", "cuda")
    nb = m.workspace_size(m.WS_FORWARD, T, 256, k, H, 512) + m.workspace_size(m.WS_SHARED, T, 1, 1, H, 512)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    m.moe_q4_workspace_init(ws)
    lg = torch.empty((T, 256), dtype=torch.int16, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    x_out = torch.empty_like(x)
    m.moe_q4_forward_ex(x, yprev, x_out, wr, None, lg, T, k, lay, sx, idx, gate, y, ws)
    torch.cuda.synchronize()
    xin = oracle.residual(np_u16(x), yprev.cpu().numpy())
    assert np.array_equal(np_u16(x_out), xin)
    _, ir, _, yr = oracle.moe_layer(lay, xin, T, k, router_w=np_u16(wr))
    assert np.array_equal(idx.cpu().numpy(), ir)
    yr = oracle.shared(H, 512, *[t.cpu().numpy() for t in sx.tensors()], xin, T, y_in=yr)
    assert_close(y.cpu().numpy(), yr, "fp8 + shared + residual")


# ------------------------------------------------------------------ prefill

def hip_experts(mode, lay, x, idx, gate, k):
    import quantized_moe_expert_amd as m
    T = x.shape[0]
    kind = m.WS_DECODE if mode == "decode" else m.WS_PREFILL
    ws = torch.empty(max(m.workspace_size(kind, T, lay.num_experts, k, lay.hidden, lay.inter), 256),
                     dtype=torch.uint8, device="cuda")
    y = torch.full((T, lay.hidden), float("nan"), dtype=torch.float32, device="cuda")
    (m.moe_q4_decode if mode == "decode" else m.moe_q4_prefill)(x, idx, gate, T, k, lay, y, ws)
    torch.cuda.synchronize()
    return y


def test_fp8_prefill_recipe_zipf_all_tokens():
    """512 tokens with Zipf(1.1) expert popularity (the prefill recipe) on the FP8 layer, every token."""
    lay, _ = recipe_layer()
    T, k, E = 512, 8, 256
    x = synth.bf16_bits(synth.normal((T, 2048), 1.0, 0, "fp8/px", "cuda"))
    lg = synth.zipf_logits(T, E, 1.1, 0, "cuda")
    _, idx, gate = hip_route(None, None, lg, T, 2048, E, k)
    y = hip_experts("prefill", lay, x, idx, gate, k).cpu().numpy()
    _, ir, _, yr = oracle.moe_layer(lay, np_u16(x), T, k, logits=np_u16(lg))
    assert np.array_equal(idx.cpu().numpy(), ir)
    r, a = assert_close(y, yr, "fp8 prefill zipf")
    say(f"[fp8 prefill] T=512 zipf, all tokens: rel L2 {r:.2e}, max abs {a:.2e}")
    yd = hip_experts("decode", lay, x, idx, gate, k).cpu().numpy()
    assert_close(y, yd, "fp8 prefill vs decode")


def test_fp8_prefill_long_all_tokens():
    """4096 tokens, N(0,1) logits (the long-prompt recipe) on the FP8 layer, every token."""
    lay, _ = recipe_layer()
    T, k, E = 4096, 8, 256
    x = synth.bf16_bits(synth.normal((T, 2048), 1.0, 0, "fp8/lx", "cuda"))
    lg = synth.bf16_bits(synth.normal((T, E), 1.0, 0, "fp8/llg", "cuda"))
    _, idx, gate = hip_route(None, None, lg, T, 2048, E, k)
    y = hip_experts("prefill", lay, x, idx, gate, k).cpu().numpy()
    _, ir, _, yr = oracle.moe_layer(lay, np_u16(x), T, k, logits=np_u16(lg))
    assert np.array_equal(idx.cpu().numpy(), ir)
    r, a = assert_close(y, yr, "fp8 prefill long")
    say(f"[fp8 prefill] T=4096, all tokens: rel L2 {r:.2e}, max abs {a:.2e}")


@pytest.mark.parametrize("T", [1, 37, 200])
def test_fp8_prefill_ragged(T):
    H, I, E, k = 512, 256, 64, 6
    lay = synth.random_layer(E, H, I, FP8, seed=21, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 21, f"fp8/prx/{T}", "cuda"))
    lg = synth.bf16_bits(synth.normal((T, E), 1.0, 21, f"fp8/prl/{T}", "cuda"))
    _, idx, gate = hip_route(None, None, lg, T, H, E, k)
    y = hip_experts("prefill", lay, x, idx, gate, k)
    _, ir, gr, yr = oracle.moe_layer(lay, np_u16(x), T, k, logits=np_u16(lg))
    assert np.array_equal(idx.cpu().numpy(), ir)
    assert_close(y.cpu().numpy(), yr, f"fp8 prefill T={T}")


def test_fp8_prefill_zero_blocks():
    """All-zero 128 x 128 blocks (scale 0, codes 0), the first input block
    among them, in gate, up and down: the accumulator rescale skips them."""
    H, I, E, k, T = 512, 256, 4, 2, 64
    lay = synth.random_layer(E, H, I, FP8, seed=23, device="cuda")
    for e in range(E):
        lay.gate_q[e, 0:128, 0:128] = 0
        lay.gate_sm[e, 0, 0] = 0.0
        lay.up_q[e, 128:256, 256:384] = 0
        lay.up_sm[e, 1, 2] = 0.0
        lay.down_q[e, 256:384, 128:256] = 0
        lay.down_sm[e, 2, 1] = 0.0
    lay.gate_q[1, 128:256, :] = 0          # every block of a row block zero
    lay.gate_sm[1, 1, :] = 0.0
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 23, "fp8/zx", "cuda"))
    lg = synth.bf16_bits(synth.normal((T, E), 1.0, 23, "fp8/zl", "cuda"))
    _, idx, gate = hip_route(None, None, lg, T, H, E, k)
    _, ir, gr, yr = oracle.moe_layer(lay, np_u16(x), T, k, logits=np_u16(lg))
    for mode in ("prefill", "decode"):
        y = hip_experts(mode, lay, x, idx, gate, k)
        assert_close(y.cpu().numpy(), yr, f"fp8 zero blocks {mode}")
