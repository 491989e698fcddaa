"""The CPU oracle against its pins (no GPU needed).  See oracle_pins.py."""
import numpy as np
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
