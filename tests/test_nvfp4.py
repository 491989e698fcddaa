"""NVFP4 routed experts (E2M1 codes, one E4M3 scale per 16 inputs, a float32
global scale per matrix, gate and up sharing theirs) on the HIP path against
the CPU oracle, through the C ABI (needs an MI355X).

Bars: dequantised weights and expert indices bit-exact; layer outputs within
relative L2 2e-3 and max abs 1e-2 of the fp64 oracle.  Inputs: the layer
recipe (H = 2048, 256 experts, top-8, I = 512) with N(0, 0.02) weights
encoded by synth's NVFP4 round-to-nearest, at 1 and 16 tokens (decode
GEMVs) and 512 (Zipf popularity) and 4096 tokens (grouped GEMMs, every
tokens), and random codes and scales at small, ragged and extreme shapes,
with zero block scales.
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
NV = synth.FMT_NVFP4


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_expert_amd as m
    m.lib()
    return torch.device("cuda")


def dequant_check(lay, e, proj):
    import quantized_moe_expert_amd as m
    H, I = lay.hidden, lay.inter
    N, K = (H, I) if proj == 2 else (I, H)
    out = torch.empty((N, K), dtype=torch.float32, device="cuda")
    m.moe_q4_dequant(lay, e, proj, out)
    host = oracle.layer_np(lay)
    g = float(lay.global_scale[e, 1 if proj == 2 else 0])
    ref = oracle.dequant(NV, host[proj][e], host[3 + proj][e], N, K, g)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), (e, proj)


@pytest.mark.parametrize("shape", [(2, 256, 128), (2, 2048, 512), (1, 64, 2048)])
def test_dequant_nvfp4_bit_exact(shape):
    E, H, I = shape
    say(f"[dequant nvfp4] E={E} H={H} I={I}")
    lay = synth.random_layer(E, H, I, NV, seed=5, device="cuda")
    for e in range(E):
        for proj in range(3):
            dequant_check(lay, e, proj)


def test_dequant_nvfp4_every_code_and_scale():
    """All 256 code bytes against all finite E4M3 scale bytes."""
    H, I = 256, 512
    lay = synth.random_layer(1, H, I, NV, seed=6, device="cuda")
    lay.gate_q.view(-1).copy_(torch.arange(256, dtype=torch.int32).to(torch.uint8).repeat(I * H // 2 // 256).to("cuda"))
    sc = torch.tensor([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=torch.uint8)
    n = I * H // 16
    lay.gate_sm.view(-1).copy_(sc.repeat(n // len(sc) + 1)[:n].to("cuda"))
    lay.global_scale[0, 0] = 3.0e-3
    dequant_check(lay, 0, 0)


_layers = {}


def recipe_layer():
    if "r" not in _layers:
        say("[gen] nvfp4 recipe layer")
        _layers["r"] = synth.make_layer(256, 2048, 512, NV, seed=0, tag="nvfp4_layer", device="cuda")
        _layers["w"] = synth.bf16_bits(synth.normal((256, 2048), 0.02, 0, "nvfp4_layer/router", "cuda"))
    return _layers["r"], _layers["w"]


def hip_forward(lay, x, k, router_w=None, logits=None):
    import quantized_moe_expert_amd as m
    T, H, E = x.shape[0], lay.hidden, lay.num_experts
    ws = torch.zeros(max(m.workspace_size(m.WS_FORWARD, T, E, k, H, lay.inter), 256), dtype=torch.uint8,
                     device="cuda")
    m.moe_q4_workspace_init(ws)
    lg = torch.empty((T, E), dtype=torch.int16, device="cuda") if logits is None else logits.clone()
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    m.moe_q4_forward(x, None, None, router_w, None, lg, T, k, lay, idx, gate, y, ws)
    torch.cuda.synchronize()
    return y, idx


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


@pytest.mark.parametrize("T", [1, 16])
def test_nvfp4_forward_recipe(T):
    lay, wr = recipe_layer()
    x = synth.bf16_bits(synth.normal((T, 2048), 1.0, 0, f"nv/x/{T}", "cuda"))
    y, idx = hip_forward(lay, x, 8, router_w=wr)
    _, ir, _, yr = oracle.moe_layer(lay, np_u16(x), T, 8, router_w=np_u16(wr))
    assert np.array_equal(idx.cpu().numpy(), ir)
    r, a = assert_close(y.cpu().numpy(), yr, f"nvfp4 forward T={T}")
    say(f"[nvfp4 forward] T={T}: rel L2 {r:.2e}, max abs {a:.2e}")


def test_nvfp4_prefill_recipe_zipf_all_tokens():
    lay, _ = recipe_layer()
    T, k, E = 512, 8, 256
    x = synth.bf16_bits(synth.normal((T, 2048), 1.0, 0, "nv/px", "cuda"))
    lg = synth.zipf_logits(T, E, 1.1, 0, "cuda")
    _, idx, gate = hip_route(None, None, lg, T, 2048, E, k)
    y = hip_experts("prefill", lay, x, idx, gate, k).cpu().numpy()
    _, ir, _, yr = oracle.moe_layer(lay, np_u16(x), T, k, logits=np_u16(lg))
    assert np.array_equal(idx.cpu().numpy(), ir)
    r, a = assert_close(y, yr, "nvfp4 prefill zipf")
    say(f"[nvfp4 prefill] T=512 zipf, all tokens: rel L2 {r:.2e}, max abs {a:.2e}")
    yd = hip_experts("decode", lay, x, idx, gate, k).cpu().numpy()
    assert_close(y, yd, "nvfp4 prefill vs decode")


def test_nvfp4_prefill_long_all_tokens():
    lay, _ = recipe_layer()
    T, k, E = 4096, 8, 256
    x = synth.bf16_bits(synth.normal((T, 2048), 1.0, 0, "nv/lx", "cuda"))
    lg = synth.bf16_bits(synth.normal((T, E), 1.0, 0, "nv/llg", "cuda"))
    _, idx, gate = hip_route(None, None, lg, T, 2048, E, k)
    y = hip_experts("prefill", lay, x, idx, gate, k).cpu().numpy()
    _, ir, _, yr = oracle.moe_layer(lay, np_u16(x), T, k, logits=np_u16(lg))
    assert np.array_equal(idx.cpu().numpy(), ir)
    r, a = assert_close(y, yr, "nvfp4 prefill long")
    say(f"[nvfp4 prefill] T=4096, all tokens: rel L2 {r:.2e}, max abs {a:.2e}")


@pytest.mark.parametrize("mode", ["decode", "prefill"])
@pytest.mark.parametrize("T", [1, 37, 200])
def test_nvfp4_ragged(mode, T):
    H, I, E, k = 512, 256, 64, 6
    lay = synth.random_layer(E, H, I, NV, seed=21, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 21, f"nv/rx/{T}", "cuda"))
    lg = synth.bf16_bits(synth.normal((T, E), 1.0, 21, f"nv/rl/{T}", "cuda"))
    _, idx, gate = hip_route(None, None, lg, T, H, E, k)
    y = hip_experts(mode, lay, x, idx, gate, k)
    _, ir, gr, yr = oracle.moe_layer(lay, np_u16(x), T, k, logits=np_u16(lg))
    assert np.array_equal(idx.cpu().numpy(), ir)
    assert_close(y.cpu().numpy(), yr, f"nvfp4 {mode} T={T}")


@pytest.mark.parametrize("shape", [(64, 2048), (2048, 64)])
def test_nvfp4_extreme_shapes(shape):
    H, I = shape
    E, k, T = 8, 2, 5
    lay = synth.random_layer(E, H, I, NV, seed=12, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 12, f"nv/ex/{H}", "cuda"))
    lg = synth.bf16_bits(synth.normal((T, E), 1.0, 12, f"nv/exl/{H}", "cuda"))
    y, idx = hip_forward(lay, x, k, logits=lg)
    _, ir, _, yr = oracle.moe_layer(lay, np_u16(x), T, k, logits=np_u16(lg))
    assert np.array_equal(idx.cpu().numpy(), ir)
    assert_close(y.cpu().numpy(), yr, f"nvfp4 {H}x{I}")


def test_nvfp4_zero_scales():
    """Blocks whose E4M3 scale is zero (and a whole zero global) in gate, up and down."""
    H, I, E, k, T = 512, 256, 4, 2, 64
    lay = synth.random_layer(E, H, I, NV, seed=23, device="cuda")
    lay.gate_sm[:, :, 0] = 0
    lay.up_sm[:, 7, :] = 0
    lay.down_sm[:, :, 5] = 0
    lay.global_scale[2, 1] = 0.0
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 23, "nv/zx", "cuda"))
    lg = synth.bf16_bits(synth.normal((T, E), 1.0, 23, "nv/zl", "cuda"))
    _, idx, gate = hip_route(None, None, lg, T, H, E, k)
    _, ir, gr, yr = oracle.moe_layer(lay, np_u16(x), T, k, logits=np_u16(lg))
    for mode in ("prefill", "decode"):
        y = hip_experts(mode, lay, x, idx, gate, k)
        assert_close(y.cpu().numpy(), yr, f"nvfp4 zero scales {mode}")
