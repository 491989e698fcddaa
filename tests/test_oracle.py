"""The CPU oracle against its pins (no GPU needed).  See oracle_pins.py."""
import numpy as np
import torch
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin()


def test_quantizer_error_matches_pages(orc):
    """Symmetric group-128 int4 with the 20-ratio clip search on Gaussian weights
    reconstructs with ~10.3% mean relative error per matrix (drama-3-w4a16 card,
    "How it was made"); this pins the synthetic weight generator, measured
    through the oracle's dequantisation."""
    import synth
    w = synth.normal((6, 512, 2048), 0.02, 0, "pin/quant", "cpu")
    q, sm = synth.quantize(w, synth.FMT_SYM_G128, clip=True)
    errs = []
    for e in range(w.shape[0]):
        d = orc.dequant(synth.FMT_SYM_G128, q[e].numpy(), sm[e].numpy(), 512, 2048).astype(np.float64)
        ref = w[e].double().numpy()
        errs.append(np.linalg.norm(d - ref) / np.linalg.norm(ref))
    assert 0.095 < np.mean(errs) < 0.108, np.mean(errs)
    # plain round-to-nearest (one ratio) must be worse than the search
    q1, sm1 = synth.quantize(w[:1], synth.FMT_SYM_G128, clip=False)
    d1 = orc.dequant(synth.FMT_SYM_G128, q1[0].numpy(), sm1[0].numpy(), 512, 2048)
    e1 = np.linalg.norm(d1 - w[0].numpy()) / np.linalg.norm(w[0].numpy())
    assert e1 > errs[0]


def test_asym_codes_in_range_and_layout(orc):
    """Asymmetric g64 encoding round-trips through the oracle within one step per weight."""
    import synth
    w = synth.normal((64, 256), 0.02, 0, "pin/asym", "cpu")
    q, sm = synth.quantize(w, synth.FMT_ASYM_G64, clip=True)
    d = orc.dequant(synth.FMT_ASYM_G64, q.numpy(), sm.numpy(), 64, 256)
    s = np.abs(sm[..., 0].numpy().view(np.float16).astype(np.float64))
    step = np.repeat(s, 64, axis=1)
    err = np.abs(d - w.numpy())
    # clipped ends may exceed half a step; the bulk must not
    assert np.mean(err <= 0.5 * step + 1e-7) > 0.97


def test_int8_encoder_round_trip(orc):
    """The synthetic int8 symmetric g128 encoder: codes in [-127, 127], every
    group's largest weight hits +-127 and each weight is within half a step of
    its dequantised value (through the oracle's int8 dequantisation)."""
    import synth
    w = synth.normal((96, 384), 0.02, 0, "pin/int8", "cpu")
    w[3, 128:256] = 0.0  # an all-zero group
    q, s = synth.quantize_int8(w)
    qn = q.numpy()
    assert qn.dtype == np.int8 and qn.min() >= -127 and qn.max() <= 127
    amax = np.abs(qn.reshape(96, 3, 128).astype(np.int64)).max(axis=2)
    assert amax[3, 1] == 0 and (np.delete(amax.ravel(), 3 * 3 + 1) == 127).all()
    d = orc.dequant_int8(qn, s.numpy(), 96, 384).astype(np.float64)
    step = np.repeat(np.abs(s.numpy().view(np.float16).astype(np.float64)), 128, axis=1)
    assert (np.abs(d - w.double().numpy()) <= 0.5 * step * (1 + 1e-3) + 1e-12).all()


def test_fp8_encoder_round_trip(orc):
    """The synthetic block-FP8 encoder: each 128 x 128 block's largest weight
    becomes +-448 (its scale is max|w| / 448), and each weight is within half
    an E4M3 step of its dequantised value (checked through the oracle)."""
    import synth
    w = synth.normal((256, 384), 0.02, 0, "pin/fp8", "cpu")
    w[128:, 128:256] = 0.0  # an all-zero block
    q, s = synth.quantize_fp8(w)
    assert q.dtype == torch.uint8 and s.shape == (2, 3)
    assert float(s[1, 1]) == 0.0
    d = orc.dequant(synth.FMT_FP8_B128, q.numpy(), s.numpy(), 256, 384).astype(np.float64)
    v = np.array([orc.e4m3_value(b) for b in range(256)])[q.numpy()]
    blocks = np.abs(v).reshape(2, 128, 3, 128).max(axis=(1, 3))
    assert (blocks[s.numpy() > 0] == 448.0).all()
    ratio = w.double().numpy() / np.repeat(np.repeat(np.where(s.numpy() > 0, s.numpy(), 1.0), 128, 0), 128, 1)
    # half a step: 2^(e-4) for normal values (e the binade), 2^-10 below 2^-6
    step = np.where(np.abs(v) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 1e-30))) - 4), 2.0 ** -10)
    assert (np.abs(ratio - v) <= step * (1 + 1e-6) + 1e-12).all()
    assert np.allclose(d, v * np.repeat(np.repeat(s.numpy().astype(np.float64), 128, 0), 128, 1))


def test_nvfp4_encoder_round_trip(orc):
    """The synthetic NVFP4 encoder: gate and up share a global scale (the
    larger amax / (6 * 448)), each weight is within half an E2M1 step (of
    the grid around it) of its dequantised value, and each 16-block's
    largest weight dequantises to at least 4 times its scale."""
    import synth
    lay = synth.make_layer(2, 256, 128, synth.FMT_NVFP4, seed=0, tag="pin/nvfp4")
    g = lay.global_scale.numpy().astype(np.float64)
    for e in range(2):
        w = {n: synth.normal(shape, 0.02, 0, f"pin/nvfp4/{n}/{e}", "cpu").double().numpy()
             for n, shape in (("gate", (128, 256)), ("up", (128, 256)), ("down", (256, 128)))}
        assert np.isclose(g[e, 0], max(np.abs(w["gate"]).max(), np.abs(w["up"]).max()) / 2688, rtol=1e-6)
        assert np.isclose(g[e, 1], np.abs(w["down"]).max() / 2688, rtol=1e-6)
        for name, q, sb, gi, (N, K) in (("gate", lay.gate_q, lay.gate_sm, 0, (128, 256)),
                                        ("up", lay.up_q, lay.up_sm, 0, (128, 256)),
                                        ("down", lay.down_q, lay.down_sm, 1, (256, 128))):
            d = orc.dequant(synth.FMT_NVFP4, q[e].numpy(), sb[e].numpy(), N, K, float(g[e, gi])).astype(np.float64)
            s = np.array([orc.e4m3_value(b) for b in sb[e].numpy().ravel()]).reshape(N, K // 16) * g[e, gi]
            s = np.repeat(s, 16, axis=1)
            a = np.abs(w[name]) / s
            half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
            assert (np.abs(w[name] - d) <= (half + 1e-6) * s).all(), name
            blk = (np.abs(d) / s).reshape(N, K // 16, 16).max(axis=2)
            assert (blk >= 4).all(), name


def test_tie_logits_put_ties_at_rank_k(orc):
    """The routing tie tests' input generator does what they rely on: in every
    token the oracle's k-th pick belongs to a tie (a signed zero, or NaN /
    -inf) that goes on past rank k, so a wrong tie rule picks another index."""
    from tie_cases import NEG_INF, tie_logits
    for T, E, k in ((64, 256, 8), (40, 16, 2), (9, 9, 5)):
        lg = tie_logits(T, E, k, seed=1 + E)
        ir, _ = orc.topk(lg, T, E, k)
        for t in range(T):
            row = lg[t]
            zero = (row & 0x7fff) == 0
            low = (row == NEG_INF) | ((row & 0x7fff) > 0x7f80)
            cls = zero if zero[ir[t, k - 1]] else low
            assert cls[ir[t, k - 1]], (T, E, k, t)
            unpicked = np.setdiff1d(np.flatnonzero(cls), ir[t])
            assert unpicked.size > 0, (T, E, k, t)
            # both signs (or both NaN and -inf) occur in the tie in some token
        kinds = set()
        for t in range(T):
            v = lg[t, ir[t, k - 1]]
            kinds.add("-0" if v == 0x8000 else "+0" if v == 0 else "-inf" if v == NEG_INF else "nan")
        assert kinds == {"-0", "+0", "-inf", "nan"}, kinds
