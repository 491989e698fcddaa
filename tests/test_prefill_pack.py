"""The prefill copy of the routed weights (moe_q4_prefill_pack) on the HIP
path, through the C ABI (needs an MI355X).

Bars:
  * the copy is bit-exact against its layout as the public header states it,
    built here on the host from the canonical arrays by reshapes and
    transposes, and for the int4 formats each row's power-of-two lift and its
    scale words times 2^L;
  * the prefill path gives bit-identical outputs with and without the copy,
    and with it stays within relative L2 2e-3 and max abs 1e-2 of the fp64
    oracle.
Formats: int4 asymmetric g64, symmetric g128, block FP8 and NVFP4.  Shapes: two column
blocks and several K-steps per GEMM at small sizes with ragged token counts;
the 512-token Zipf layer and the 4096-token symmetric layer at full size
(all tokens bit-identical, and all against the oracle).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import assert_close, hip_experts, hip_route, np_u16, oracle_y

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


def _host_bytes(t):
    return t.detach().cpu().contiguous().numpy().view(np.uint8).reshape(-1)


def _tiles_codes(rows, ncb, block_rows, K):
    """[E][N][K/2] codes -> [E][ncb][K/64][block_rows][32], halves of the
    32-byte chunk swapped in rows whose bit 3 is set."""
    E = rows.shape[0]
    t = rows.reshape(E, ncb, block_rows, K // 64, 2, 16).transpose(0, 1, 3, 2, 4, 5).copy()
    sw = ((np.arange(block_rows) >> 3) & 1).astype(bool)
    t[:, :, :, sw] = t[:, :, :, sw][:, :, :, :, ::-1]
    return t.reshape(-1)


def _tiles_codes_fp8(rows, ncb, block_rows, K):
    """[E][N][K] FP8 codes -> [E][ncb][K/64][block_rows][64], the 16-byte
    quarter q of a row's 64 bytes stored at q ^ ((row >> 2) & 3)."""
    E = rows.shape[0]
    t = rows.reshape(E, ncb, block_rows, K // 64, 4, 16).transpose(0, 1, 3, 2, 4, 5)
    out = np.empty_like(t)
    sel = (np.arange(block_rows) >> 2) & 3
    for q in range(4):
        for x in range(4):
            r = sel == x
            out[:, :, :, r, q ^ x] = t[:, :, :, r, q]
    return out.reshape(-1)


# canonical scale entries: (inputs per entry, bytes per entry)
ENTRY = {synth.FMT_ASYM_G64: (64, 4), synth.FMT_SYM_G128: (128, 2), synth.FMT_NVFP4: (16, 1)}


def _step_words(sm, E, N, K, fmt):
    """[E][N][K/64]: for each row and K-step j, the 4-byte-aligned word of the
    canonical scale array that holds the row's entry for input 64 j."""
    words = _host_bytes(sm).view(np.uint32)
    G, esz = ENTRY[fmt]
    row = np.arange(E * N)[:, None]
    j = np.arange(K // 64)[None, :]
    byte = (row * (K // G) + (64 * j) // G) * esz
    return words[byte // 4].reshape(E, N, K // 64)


def _row_lifts(sm, E, N, K, fmt):
    """[E][N] int: a row's power-of-two lift L = 10 - floor(log2 A), A the
    largest magnitude among its f16 scales (and mins), 0 for A = 0."""
    halves = _host_bytes(sm).view(np.float16).reshape(E, N, -1).astype(np.float64)
    a = np.max(np.abs(halves), axis=2)
    lg = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 10 - lg, 0).astype(np.int64)


def _lift_words(words, lifts):
    """Both f16 halves of each uint32 word times 2^L of its row (one rounding)."""
    w = np.ascontiguousarray(words)
    h = w.view(np.float16).reshape(*w.shape, 2).astype(np.float64)
    out = np.ldexp(h, lifts[..., None, None]).astype(np.float16)
    return np.ascontiguousarray(out).view(np.uint32).reshape(w.shape)


def expected_pack(lay):
    E, H, I, fmt = lay.num_experts, lay.hidden, lay.inter, lay.fmt
    if fmt == synth.FMT_FP8_B128:
        gq = _host_bytes(lay.gate_q).reshape(E, I, H)
        uq = _host_bytes(lay.up_q).reshape(E, I, H)
        dq = _host_bytes(lay.down_q).reshape(E, H, I)
        gu = np.concatenate([gq.reshape(E, I // 128, 128, H), uq.reshape(E, I // 128, 128, H)], axis=2)
        out = np.concatenate([_tiles_codes_fp8(gu, I // 128, 256, H), _tiles_codes_fp8(dq, H // 256, 256, I)])
        assert out.size == 3 * E * I * H
        return out
    gq = _host_bytes(lay.gate_q).reshape(E, I, H // 2)
    uq = _host_bytes(lay.up_q).reshape(E, I, H // 2)
    dq = _host_bytes(lay.down_q).reshape(E, H, I // 2)
    # gate|up: column block c = gate rows 128c.. then the same up rows
    gu = np.concatenate([gq.reshape(E, I // 128, 128, H // 2), uq.reshape(E, I // 128, 128, H // 2)], axis=2)
    gu_q = _tiles_codes(gu, I // 128, 256, H)
    d_q = _tiles_codes(dq, H // 256, 256, I)
    gw = _step_words(lay.gate_sm, E, I, H, fmt)
    uw = _step_words(lay.up_sm, E, I, H, fmt)
    dw = _step_words(lay.down_sm, E, H, I, fmt)
    int4 = fmt in (synth.FMT_ASYM_G64, synth.FMT_SYM_G128)
    if int4:  # scale words lifted by the row's power of two
        gl = _row_lifts(lay.gate_sm, E, I, H, fmt)
        ul = _row_lifts(lay.up_sm, E, I, H, fmt)
        dl = _row_lifts(lay.down_sm, E, H, I, fmt)
        gw, uw, dw = _lift_words(gw, gl), _lift_words(uw, ul), _lift_words(dw, dl)
    gw = gw.reshape(E, I // 128, 128, H // 64)
    uw = uw.reshape(E, I // 128, 128, H // 64)
    gu_s = np.concatenate([gw, uw], axis=2).transpose(0, 1, 3, 2).reshape(-1)
    d_s = dw.reshape(E, H // 256, 256, I // 64).transpose(0, 1, 3, 2).reshape(-1)
    parts = [gu_q, np.ascontiguousarray(gu_s).view(np.uint8), d_q, np.ascontiguousarray(d_s).view(np.uint8)]
    if int4:  # the lifts: gate|up [E][I/128][256] (gate rows, then up rows), down [E][H/256][256]
        gul = np.concatenate([gl.reshape(E, I // 128, 128), ul.reshape(E, I // 128, 128)], axis=2)
        parts += [gul.astype(np.int8).reshape(-1).view(np.uint8), dl.astype(np.int8).reshape(-1).view(np.uint8)]
    out = np.concatenate(parts)
    assert out.size == 27 * E * I * H // 16 + (2 * E * I + E * H if int4 else 0)
    return out


FORMATS = [synth.FMT_ASYM_G64, synth.FMT_SYM_G128, synth.FMT_FP8_B128, synth.FMT_NVFP4]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", [(3, 512, 256), (2, 256, 128), (1, 2048, 512)])
def test_pack_bytes(fmt, shape):
    import quantized_moe_expert_amd as m
    E, H, I = shape
    say(f"[pack bytes] fmt={fmt} E={E} H={H} I={I}")
    lay = synth.random_layer(E, H, I, fmt, seed=21, device="cuda")
    pk = m.prefill_pack(lay)
    torch.cuda.synchronize()
    got = pk.cpu().numpy()
    exp = expected_pack(lay)
    assert got.size == exp.size
    bad = np.flatnonzero(got != exp)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:4]}"


def _both(lay, x, idx, gate, k):
    import quantized_moe_expert_amd as m
    y0 = hip_experts("prefill", lay, x, idx, gate, k).clone()
    pk = m.prefill_pack(lay)
    y1 = hip_experts("prefill", m.layer_struct(lay, pack=pk), x, idx, gate, k)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), "outputs with the copy differ"
    return y1


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("T", [1, 37, 200])
def test_prefill_with_pack_ragged(fmt, T):
    """Ragged token counts on a 64-expert layer (two column blocks per GEMM)
    with random codes and scales."""
    H, I, E, k = 512, 256, 64, 6
    say(f"[pack ragged] fmt={fmt} T={T}")
    lay = synth.random_layer(E, H, I, fmt, seed=9, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 9, f"pk/x/{T}", "cuda"))
    wr = synth.bf16_bits(synth.normal((E, H), 0.05, 9, "pk/w", "cuda"))
    lg, idx, gate = hip_route(x, wr, None, T, H, E, k)
    lr = oracle.router(np_u16(x), np_u16(wr), T, H, E)
    ir, gr = oracle.topk(lr, T, E, k)
    assert np.array_equal(idx.cpu().numpy(), ir)
    y = _both(lay, x, idx, gate, k)
    yr = oracle_y(lay, np_u16(x), ir, gr, k)
    assert_close(y.cpu().numpy(), yr, f"pack ragged fmt={fmt} T={T}")


@pytest.mark.parametrize("cfg,fmt", [(3, None), (3, synth.FMT_NVFP4), (3, synth.FMT_FP8_B128), (5, None),
                                     (5, synth.FMT_FP8_B128)])
def test_prefill_with_pack_full_size(cfg, fmt):
    """The 512-token Zipf layer (int4 asym, NVFP4, block FP8) and the
    4096-token layer (int4 sym, block FP8): every output bit-identical with
    the copy, and every token against the oracle."""
    say(f"[pack full] config {cfg} fmt={fmt}")
    case = synth.make_case(cfg, device="cuda", fmt=fmt)
    lay = case.layers[0]
    lg, idx, gate = hip_route(None, None, case.logits, case.T, case.H, case.E, case.k)
    y = _both(lay, case.x, idx, gate, case.k)
    ir, gr = oracle.topk(np_u16(case.logits), case.T, case.E, case.k)
    assert np.array_equal(idx.cpu().numpy(), ir)
    yr = oracle_y(lay, np_u16(case.x), ir, gr, case.k)
    r, a = assert_close(y.cpu().numpy(), yr, f"pack config {cfg}")
    say(f"[pack full] config {cfg}: rel L2 {r:.2e}, max abs {a:.2e}")


def test_forward_with_pack():
    """moe_q4_forward through MoeQ4Layer(pack_prefill=True) on the prefill
    path (T > 64) equals the layer without the copy."""
    import quantized_moe_expert_amd as m
    case = synth.make_case(3, device="cuda", T=300)
    lay = case.layers[0]
    a = m.MoeQ4Layer(lay, case.k, case.T, mode="prefill")
    b = m.MoeQ4Layer(lay, case.k, case.T, mode="prefill", pack_prefill=True)
    ya = a.forward(case.x, logits=case.logits).clone()
    yb = b.forward(case.x, logits=case.logits)
    torch.cuda.synchronize()
    assert torch.equal(ya.view(torch.int32), yb.view(torch.int32))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("H,I", [(256, 128), (2048, 128), (256, 2048)])
def test_prefill_extreme_shapes(fmt, H, I):
    """The smallest and largest K loops of the grouped GEMMs (2 K-steps in
    the down GEMM at I = 128, more stages in flight than K-steps; 32 at
    2048) and single column blocks, with 150 rows per expert on average
    (full and partial tiles) over the multi-block grouping: outputs against
    the oracle, and bit-identical with and without the prefill copy."""
    T, E, k = 600, 8, 2
    say(f"[pack extreme] fmt={fmt} H={H} I={I}")
    lay = synth.random_layer(E, H, I, fmt, seed=17, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 17, f"pkx/x/{H}", "cuda"))
    logits = synth.bf16_bits(synth.normal((T, E), 1.0, 17, f"pkx/l/{H}/{I}", "cuda"))
    lg, idx, gate = hip_route(None, None, logits, T, H, E, k)
    ir, gr = oracle.topk(np_u16(logits), T, E, k)
    assert np.array_equal(idx.cpu().numpy(), ir)
    y = _both(lay, x, idx, gate, k)
    assert_close(y.cpu().numpy(), oracle_y(lay, np_u16(x), ir, gr, k), f"pack extreme fmt={fmt} H={H} I={I}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_prefill_paired_down_schedule(fmt):
    """About 300 rows per expert over 20 experts (two full 128-row tiles and a
    partial one of about two subtiles each): the down GEMM's schedule pairs
    16 experts' last full tiles with their partial tiles in two blocks of 8
    and leaves 4 experts unpaired.  Outputs against the oracle on every
    token, and bit-identical with and without the prefill copy."""
    T, H, I, E, k = 1500, 512, 256, 20, 4
    say(f"[paired schedule] fmt={fmt}")
    lay = synth.random_layer(E, H, I, fmt, seed=23, device="cuda")
    x = synth.bf16_bits(synth.normal((T, H), 1.0, 23, "pair/x", "cuda"))
    logits = synth.bf16_bits(synth.normal((T, E), 1.0, 23, "pair/l", "cuda"))
    lg, idx, gate = hip_route(None, None, logits, T, H, E, k)
    ir, gr = oracle.topk(np_u16(logits), T, E, k)
    assert np.array_equal(idx.cpu().numpy(), ir)
    cnt = np.bincount(ir.ravel(), minlength=E)
    paired = int(np.sum((cnt > 128) & (cnt % 128 != 0)))
    assert paired >= 16 and paired % 8 != 0, cnt  # whole blocks and leftovers
    y = _both(lay, x, idx, gate, k)
    assert_close(y.cpu().numpy(), oracle_y(lay, np_u16(x), ir, gr, k), f"paired schedule fmt={fmt}")
