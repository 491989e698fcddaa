"""The f16 intermediates of both expert paths across magnitudes, against the
oracle (needs an MI355X).

The decode GEMVs take h in f16 (each row scaled by a power of two); the
prefill GEMMs run f16 matrix cores on x (each row scaled by a power of two),
on weights dequantised to f16, on h and on each routed row's down output z.
None of that may depend on the scale of the inputs: activations x 2^-10,
x 2^-4, x 2^4 and x 2^7 (|h| up to about 2^16), int4 group scales
log-uniform over [2^-16, 2^-4] and over [2^-16, 2^-10] (every group below
2^-10), block-FP8 scales and NVFP4 globals log-uniform over a wide range.
Every weight format, decode and prefill (with and without the prefill copy
of the weights).  The shared expert likewise, on both of its paths (see
test_shared_expert_magnitudes).  Bar: rel L2 <= 2e-3; max abs <= 1e-2 times the output's
largest magnitude when that exceeds 1.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import assert_close, hip_experts, hip_route, np_u16

pytestmark = pytest.mark.gpu

FMTS = [synth.FMT_ASYM_G64, synth.FMT_SYM_G128, synth.FMT_FP8_B128, synth.FMT_NVFP4]
E, H, I, K = 32, 512, 256, 4
# (name, log2 of the activation scale, log2 scale range of the weights or None)
CASES = [("x2^-10", -10, None), ("x2^-4", -4, None), ("x2^4", 4, None), ("x2^7", 7, None),
         ("scales 2^-16..2^-4", 0, (-16, -4)), ("scales 2^-16..2^-10", 0, (-16, -10)),
         ("scales 2^-16..2^-10, x2^-4", -4, (-16, -10))]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_expert_amd as m
    m.lib()


def _wide_layer(fmt, log2s):
    if log2s is None:
        return synth.random_layer(E, H, I, fmt, seed=41, device="cuda", tag="mag")
    lo, hi = log2s
    if fmt == synth.FMT_FP8_B128:      # block scales: codes reach 448, so shift the range down
        lo, hi = lo - 6, hi - 6
    if fmt == synth.FMT_NVFP4:         # globals: block scales reach 448 and codes 6
        lo, hi = lo - 8, hi - 8
    return synth.random_layer(E, H, I, fmt, seed=41, device="cuda", tag="mag", log2_scale=(lo, hi))


@pytest.mark.parametrize("mode,T", [("decode", 16), ("prefill", 96), ("prefill", 600), ("prefill_pack", 96),
                                    ("prefill_pack", 600)])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_magnitudes(case, fmt, mode, T):
    import quantized_moe_expert_amd as m
    name, xs, log2s = case
    say(f"[magnitudes] {name} fmt={fmt} {mode} T={T}")
    lay = _wide_layer(fmt, log2s)
    x = synth.bf16_bits(synth.normal((T, H), 2.0 ** xs, 41, f"mag/x/{T}", "cuda"))
    logits = synth.bf16_bits(synth.normal((T, E), 1.0, 41, f"mag/l/{T}", "cuda"))
    _, idx, gate = hip_route(None, None, logits, T, H, E, K)
    ir, gr = oracle.topk(np_u16(logits), T, E, K)
    assert np.array_equal(idx.cpu().numpy(), ir)
    run = lay
    if mode == "prefill_pack":
        pack = m.prefill_pack(lay)
        run = m.layer_struct(lay, pack=pack)
    y = hip_experts("decode" if mode == "decode" else "prefill", lay if mode != "prefill_pack" else run, x, idx,
                    gate, K)
    torch.cuda.synchronize()
    yr = oracle.experts(fmt, E, H, I, *oracle.layer_np(lay), np_u16(x), ir, gr, T, K,
                        global_scale=oracle.layer_global(lay))
    assert np.all(np.isfinite(yr))
    r, a = assert_close(y.cpu().numpy(), yr, f"{name} fmt={fmt} {mode}", abs_scaled=True)
    say(f"[magnitudes] {name} fmt={fmt} {mode}: rel L2 {r:.2e} max abs {a:.2e} (|y| max {np.max(np.abs(yr)):.2e})")


@pytest.mark.parametrize("mode,T", [("decode", 16), ("prefill", 96), ("prefill", 600), ("prefill_pack", 600)])
@pytest.mark.parametrize("fmt", FMTS)
def test_magnitudes_mixed_tokens(fmt, mode, T):
    """Tokens of one call at scales 2^-10 to 2^9 (each token its own): the rows of a prefill tile then differ
    by up to 2^19 in |x| and 2^38 in |h|, while the GEMMs' h and z exponents are shared over a tile's rows per
    block of columns (after each row's own 2^-2e).  Every token's row must meet the bar on its own."""
    import quantized_moe_expert_amd as m
    say(f"[magnitudes mixed] fmt={fmt} {mode} T={T}")
    lay = _wide_layer(fmt, None)
    row = torch.tensor([2.0 ** (-10 + (7 * t) % 20) for t in range(T)], device="cuda")[:, None]
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 53, f"mag/xm/{T}", "cuda") * row)
    logits = synth.bf16_bits(synth.normal((T, E), 1.0, 53, f"mag/lm/{T}", "cuda"))
    _, idx, gate = hip_route(None, None, logits, T, H, E, K)
    ir, gr = oracle.topk(np_u16(logits), T, E, K)
    assert np.array_equal(idx.cpu().numpy(), ir)
    pack = m.prefill_pack(lay) if mode == "prefill_pack" else None  # kept alive through the call
    run = m.layer_struct(lay, pack=pack) if pack is not None else lay
    y = hip_experts("decode" if mode == "decode" else "prefill", run, x, idx, gate, K)
    torch.cuda.synchronize()
    yr = oracle.experts(fmt, E, H, I, *oracle.layer_np(lay), np_u16(x), ir, gr, T, K,
                        global_scale=oracle.layer_global(lay))
    yg = y.cpu().numpy()
    assert_close(yg, yr, f"mixed fmt={fmt} {mode}", abs_scaled=True)
    worst = 0.0
    for t in range(T):
        r, _ = assert_close(yg[t], yr[t], f"mixed fmt={fmt} {mode} token {t}", abs_scaled=True)
        worst = max(worst, r)
    say(f"[magnitudes mixed] fmt={fmt} {mode}: worst per-token rel L2 {worst:.2e}")


# ------------------------------------------------------------ shared expert

def _host(sx):
    return [t.cpu().numpy() for t in sx.tensors()]


@pytest.mark.parametrize("fused", [False, True], ids=["alone", "in_layer"])
@pytest.mark.parametrize("T", [1, 16, 100])
@pytest.mark.parametrize("xs", [-10, -4, 4, 9, "mix"], ids=lambda v: f"x2^{v}")
def test_shared_expert_magnitudes(xs, T, fused):
    """The shared expert at activation scales 2^9 (|h| far above f16's 65504) and 2^-10 (h near f16's
    subnormals).  Up to 64 tokens (GEMV path, its own launches or its items inside the layer's decode
    launches) h is kept in fp32 and each token's row is scaled by a power of two before the f16 down
    product; from 65 tokens (matrix-core GEMMs, after the routed GEMMs of a prefill layer) h is stored in
    f16 scaled per row by 2^-2e and per 128-column block by a power of two, both taken off in the down
    GEMM.  "mix" gives each token its own scale, 2^-10 to 2^9, so the rows of one GEMM tile differ by up
    to 2^38 in |h|.  Every case must meet the bar."""
    import quantized_moe_expert_amd as m
    Hs, Is = 512, 256
    say(f"[magnitudes shared] x2^{xs} T={T} fused={fused}")
    sx = synth.random_shared(Hs, Is, seed=43, device="cuda", tag="mag_shared")
    if xs == "mix":
        row = torch.tensor([2.0 ** (-10 + (7 * t) % 20) for t in range(T)], device="cuda")[:, None]
        x = synth.bf16_bits(synth.normal((T, Hs), 1.0, 43, f"mag/sx/{T}", "cuda") * row)
    else:
        x = synth.bf16_bits(synth.normal((T, Hs), 2.0 ** xs, 43, f"mag/sx/{T}", "cuda"))
    x_np = np_u16(x)
    if not fused:
        ws = torch.empty(max(m.workspace_size(m.WS_SHARED, T, 1, 1, Hs, Is), 256), dtype=torch.uint8,
                         device="cuda")
        y = torch.full((T, Hs), float("nan"), dtype=torch.float32, device="cuda")
        m.moe_q4_shared(x, T, sx, y, 0, ws)
        torch.cuda.synchronize()
        yr = oracle.shared(Hs, Is, *_host(sx), x_np, T)
    else:
        # the layer's routed experts with the same inner size, so the shared items run in its launches
        lay = synth.random_layer(E, Hs, Is, synth.FMT_ASYM_G64, seed=43, device="cuda", tag="mag_shared_l")
        logits = synth.bf16_bits(synth.normal((T, E), 1.0, 43, f"mag/sl/{T}", "cuda"))
        nb = m.workspace_size(m.WS_FORWARD, T, E, K, Hs, Is) + m.workspace_size(m.WS_SHARED, T, 1, 1, Hs, Is)
        ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device="cuda")
        m.moe_q4_workspace_init(ws)
        idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
        gate = torch.empty((T, K), dtype=torch.float32, device="cuda")
        y = torch.full((T, Hs), float("nan"), dtype=torch.float32, device="cuda")
        m.moe_q4_forward_ex(x, None, None, None, None, logits.clone(), T, K, lay, sx, idx, gate, y, ws)
        torch.cuda.synchronize()
        _, ir, gr, yl = oracle.moe_layer(lay, x_np, T, K, logits=np_u16(logits))
        assert np.array_equal(idx.cpu().numpy(), ir)
        yr = oracle.shared(Hs, Is, *_host(sx), x_np, T, y_in=yl)
    assert np.all(np.isfinite(yr))
    yg = y.cpu().numpy()
    r, a = assert_close(yg, yr, f"shared x2^{xs} T={T} fused={fused}", abs_scaled=True)
    if xs == "mix":  # the small tokens are invisible in the whole output's norms: each row on its own
        for t in range(T):
            assert_close(yg[t], yr[t], f"shared mix T={T} fused={fused} token {t}", abs_scaled=True)
    say(f"[magnitudes shared] x2^{xs}: rel L2 {r:.2e} max abs {a:.2e} (|y| max {np.max(np.abs(yr)):.2e})")


@pytest.mark.parametrize("T", [16, 100, 300])
def test_shared_expert_magnitudes_wide_inner(T):
    """Inner size 2048: the GEMV path stages 2048-wide h rows, and the GEMM path keeps 16 exponent bytes
    per token (one per 128 columns of h) and folds 16 block factors into the down GEMM's scales; per-token
    activation scales 2^-10 to 2^9, each row checked on its own."""
    import quantized_moe_expert_amd as m
    Hs, Is = 256, 2048
    say(f"[magnitudes shared wide] T={T}")
    sx = synth.random_shared(Hs, Is, seed=47, device="cuda", tag="mag_shared_wide")
    row = torch.tensor([2.0 ** (-10 + (5 * t) % 20) for t in range(T)], device="cuda")[:, None]
    x = synth.bf16_bits(synth.normal((T, Hs), 1.0, 47, f"mag/sxw/{T}", "cuda") * row)
    ws = torch.empty(max(m.workspace_size(m.WS_SHARED, T, 1, 1, Hs, Is), 256), dtype=torch.uint8, device="cuda")
    y = torch.full((T, Hs), float("nan"), dtype=torch.float32, device="cuda")
    m.moe_q4_shared(x, T, sx, y, 0, ws)
    torch.cuda.synchronize()
    yr = oracle.shared(Hs, Is, *_host(sx), np_u16(x), T)
    yg = y.cpu().numpy()
    assert_close(yg, yr, f"shared wide T={T}", abs_scaled=True)
    for t in range(T):
        assert_close(yg[t], yr[t], f"shared wide T={T} token {t}", abs_scaled=True)
