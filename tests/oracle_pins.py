"""Pins of the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle currently bound
in the ``oracle`` module disagrees with its pin.  ``test_oracle.py`` runs them
against the real oracle; ``test_oracle_mutants.py`` runs them against copies of
the oracle with one planted mistake each and requires some pin to fail.

What pins what:
  * binary16 / bfloat16 decoding and bf16 rounding: numpy's float16 and
    torch's bfloat16 conversions (library routines), on every bit pattern or
    on a wide sample plus the halfway cases;
  * dequantisation: hand-packed rows with hand-worked values
    (tests/golden/dequant_cases.txt, dequant_fp8_cases.txt) and an
    independent numpy unpacking (torch's float8_e4m3fn decoding for FP8);
  * E4M3 decoding: torch's float8_e4m3fn conversion on all 256 patterns;
  * E2M1 and NVFP4: hand-worked rows (tests/golden/dequant_nvfp4_cases.txt),
    a hand-listed value table in numpy for random rows, the one-expert dense
    MLP and brute force with global scales;
  * router logits: numpy float64 matrix product, rounded by torch;
  * top-k: brute force, a full stable sort of every token's logits;
  * gates: scipy's softmax over all experts renormalised over the selected,
    sum to one, the k = 1 and k = E special cases;
  * grouping: numpy's stable argsort and the permutation invariants;
  * expert MLP + combine: dense float64 numpy matmuls with scipy's logistic
    function, the one-expert top-1 layer as a plain SwiGLU MLP, and gate
    linearity (two identical experts selected together equal one);
  * int8 dequantisation: hand-written rows with hand-worked values
    (tests/golden/dequant_int8_cases.txt) and numpy's own int8 and float16
    decoding;
  * shared expert: dense float64 numpy matmuls with scipy's logistic
    function (with and without a given y_in, on a token subset), and a
    routed one-expert top-1 layer of the same weights when every code fits
    int4 symmetric;
  * the synthetic quantiser: relative reconstruction error of symmetric
    group-128 clip-searched int4 on Gaussian weights, 10.3% on the pages
    (drama-3-w4a16 card, "How it was made").
"""
from __future__ import annotations

import os

import numpy as np
import scipy.special
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers

def np_codes(q: np.ndarray, N: int, K: int) -> np.ndarray:
    """uint8 [N][K/2] -> int codes [N][K] (low nibble = even k), by numpy bit ops."""
    q = np.asarray(q, dtype=np.uint8).reshape(N, K // 2)
    out = np.empty((N, K), dtype=np.int64)
    out[:, 0::2] = q & 0x0F
    out[:, 1::2] = q >> 4
    return out


def np_dequant64(fmt: int, q, sm, N: int, K: int) -> np.ndarray:
    """Independent float64 dequantisation using numpy's float16 decoder
    (torch's float8_e4m3fn decoder for FP8 codes)."""
    if fmt == oracle.FMT_FP8_B128:
        v = torch.from_numpy(np.asarray(q, dtype=np.uint8).reshape(N, K).copy()).view(torch.float8_e4m3fn)
        s = np.asarray(sm, dtype=np.float32).reshape(N // 128, K // 128).astype(np.float64)
        return v.double().numpy() * np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)
    codes = np_codes(q, N, K).astype(np.float64)
    g = 64 if fmt == oracle.FMT_ASYM_G64 else 128
    sm = np.asarray(sm).view(np.uint16).view(np.float16).astype(np.float64)
    if fmt == oracle.FMT_ASYM_G64:
        sm = sm.reshape(N, K // g, 2)
        s = np.repeat(sm[:, :, 0], g, axis=1)
        m = np.repeat(sm[:, :, 1], g, axis=1)
        return codes * s + m
    s = np.repeat(sm.reshape(N, K // g), g, axis=1)
    return (codes - 8.0) * s


def torch_bf16_bits(a) -> np.ndarray:
    t = torch.from_numpy(np.asarray(a, dtype=np.float32).copy())
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def rand_bf16(rng, shape, std=1.0) -> np.ndarray:
    return torch_bf16_bits(rng.standard_normal(shape) * std)


E2M1_TABLE = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])


def np_nvfp4_64(q, sb, glob, N, K) -> np.ndarray:
    """Independent float64 NVFP4 dequantisation: a hand-listed E2M1 table and
    torch's E4M3 decoding."""
    codes = np_codes(q, N, K)
    s = torch.from_numpy(np.asarray(sb, dtype=np.uint8).reshape(N, K // 16).copy()).view(torch.float8_e4m3fn)
    return E2M1_TABLE[codes] * np.repeat(s.double().numpy(), 16, axis=1) * float(glob)


def rand_layer(rng, E, H, I, fmt):
    """Random codes and f16 scales/mins of plausible magnitude (numpy arrays)."""
    g = 64 if fmt == oracle.FMT_ASYM_G64 else 128
    mats = {}
    if fmt == oracle.FMT_NVFP4:
        for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            mats[name + "_q"] = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
            mats[name + "_sm"] = rng.integers(0x28, 0x41, size=(E, N, K // 16), dtype=np.uint8)
        mats["global"] = (rng.random((E, 2)) * 0.004 + 0.004).astype(np.float32)
        return mats
    if fmt == oracle.FMT_FP8_B128:
        for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            q = rng.integers(0, 256, size=(E, N, K), dtype=np.uint8)
            q[(q & 0x7F) == 0x7F] -= 1  # no NaN codes
            mats[name + "_q"] = q
            mats[name + "_sm"] = (rng.random((E, N // 128, K // 128)) * 1e-4 + 5e-5).astype(np.float32)
        return mats
    for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        mats[name + "_q"] = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
        s = (rng.random((E, N, K // g)) * 0.004 + 0.002).astype(np.float16)
        if fmt == oracle.FMT_ASYM_G64:
            m = (-(rng.random((E, N, K // g)) * 0.03 + 0.015)).astype(np.float16)
            mats[name + "_sm"] = np.stack([s, m], axis=-1).view(np.uint16)
        else:
            mats[name + "_sm"] = s.view(np.uint16)
    return mats


def layer_args(mats):
    return [mats[n] for n in ("gate_q", "up_q", "down_q", "gate_sm", "up_sm", "down_sm")]


def glob_kw(mats):
    return {"global_scale": mats["global"]} if "global" in mats else {}


def np_expert_out(fmt, mats, e, x64, H, I):
    """o = Wd silu(Wg x) * (Wu x) in float64 with numpy matmuls and scipy's expit."""
    if fmt == oracle.FMT_NVFP4:
        g = mats["global"][e]
        wg = np_nvfp4_64(mats["gate_q"][e], mats["gate_sm"][e], g[0], I, H)
        wu = np_nvfp4_64(mats["up_q"][e], mats["up_sm"][e], g[0], I, H)
        wd = np_nvfp4_64(mats["down_q"][e], mats["down_sm"][e], g[1], H, I)
    else:
        wg = np_dequant64(fmt, mats["gate_q"][e], mats["gate_sm"][e], I, H)
        wu = np_dequant64(fmt, mats["up_q"][e], mats["up_sm"][e], I, H)
        wd = np_dequant64(fmt, mats["down_q"][e], mats["down_sm"][e], H, I)
    a = wg @ x64
    b = wu @ x64
    h = a * scipy.special.expit(a) * b
    return wd @ h


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def read_dequant_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "dequant_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, *rest = line.split()
            if head == "case":
                kv = dict(r.split("=") for r in rest[1:])
                cur = {"name": rest[0], "fmt": int(kv["fmt"]), "N": int(kv["N"]), "K": int(kv["K"])}
                cases.append(cur)
            elif head == "bytes":
                cur["bytes"] = [int(v, 16) for v in rest]
            elif head == "sm":
                cur["sm"] = [int(v, 16) for v in rest]
            elif head == "expect":
                cur["expect"] = [float(v) for v in rest]
    return cases


def read_dequant_nvfp4_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "dequant_nvfp4_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, *rest = line.split()
            if head == "case":
                kv = dict(r.split("=") for r in rest[1:])
                cur = {"name": rest[0], "N": int(kv["N"]), "K": int(kv["K"]), "global": float(kv["global"]),
                       "expect": []}
                cases.append(cur)
            elif head == "bytes":
                cur["bytes"] = [int(v, 16) for v in rest]
            elif head == "scale":
                cur["scale"] = [int(v, 16) for v in rest]
            elif head == "expect":
                cur["expect"].append([float(v) for v in rest])
    return cases


def read_dequant_fp8_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "dequant_fp8_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, *rest = line.split()
            if head == "case":
                kv = dict(r.split("=") for r in rest[1:])
                cur = {"name": rest[0], "N": int(kv["N"]), "K": int(kv["K"]), "expect": []}
                cases.append(cur)
            elif head == "bytes":
                cur["bytes"] = [int(v, 16) for v in rest]
            elif head == "scale":
                cur["scale"] = [float(v) for v in rest]
            elif head == "expect":
                cur["expect"].append([float(v) for v in rest])
    return cases


def read_dequant_int8_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "dequant_int8_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, *rest = line.split()
            if head == "case":
                kv = dict(r.split("=") for r in rest[1:])
                cur = {"name": rest[0], "N": int(kv["N"]), "K": int(kv["K"]), "expect": []}
                cases.append(cur)
            elif head == "bytes":
                cur["bytes"] = [int(v, 16) for v in rest]
            elif head == "scale":
                cur["scale"] = [int(v, 16) for v in rest]
            elif head == "expect":
                cur["expect"].append([float(v) for v in rest])
    return cases


def np_dequant_int8_64(q, s, N, K) -> np.ndarray:
    """Independent float64 int8 dequantisation (numpy's int8 and float16 decoders)."""
    q = np.asarray(q).view(np.int8).reshape(N, K).astype(np.float64)
    s = np.asarray(s).view(np.uint16).view(np.float16).astype(np.float64).reshape(N, K // 128)
    return q * np.repeat(s, 128, axis=1)


def rand_shared(rng, H, I, lo=-127, hi=127):
    """Random int8 codes in [lo, hi] and f16 scales of plausible magnitude."""
    mats = {}
    for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        mats[name + "_q"] = rng.integers(lo, hi + 1, size=(N, K)).astype(np.int8)
        mats[name + "_s"] = (rng.random((N, K // 128)) * 1.2e-3 + 2e-4).astype(np.float16).view(np.uint16)
    return mats


def shared_args(mats):
    return [mats[n] for n in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s")]


def np_shared_out(mats, x64, H, I):
    """Wd silu(Wg x) * (Wu x) in float64 (numpy matmuls, scipy's expit)."""
    wg = np_dequant_int8_64(mats["gate_q"], mats["gate_s"], I, H)
    wu = np_dequant_int8_64(mats["up_q"], mats["up_s"], I, H)
    wd = np_dequant_int8_64(mats["down_q"], mats["down_s"], H, I)
    a = wg @ x64
    return wd @ (a * scipy.special.expit(a) * (wu @ x64))


def cyc(vals, n):
    return [vals[i % len(vals)] for i in range(n)]


# -------------------------------------------------------------------- pins

def pin_f16_decode_all():
    """Every binary16 bit pattern decodes as numpy's float16 does."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_value(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_bf16_decode_all():
    """Every bfloat16 bit pattern decodes as torch's bfloat16 does."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_value(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def pin_bf16_round():
    """Round-to-nearest-even to bf16 matches torch on a wide sample and on halfway cases."""
    rng = np.random.default_rng(7)
    mant = rng.random(40000) + 1.0
    expo = rng.integers(-133, 128, size=40000)
    vals = (mant * np.exp2(expo.astype(np.float64))).astype(np.float32)
    vals *= np.where(rng.random(40000) < 0.5, -1, 1).astype(np.float32)
    # exact halfway points between neighbouring bf16 values, both parities
    hw = (rng.integers(0, 0x7f7f, size=4000, dtype=np.uint32) << 16) | 0x8000
    halfway = hw.astype(np.uint32).view(np.float32)
    special = np.array([0.0, -0.0, 3.3895314e38, 3.4028235e38, 1e-45, -1e-45, 1.1754944e-38,
                        np.inf, -np.inf, 1.0, 1.00390625, 1.01171875], dtype=np.float32)
    allv = np.concatenate([vals, halfway, special])
    got = oracle.bf16_round_array(allv)
    ref = torch_bf16_bits(allv)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} mismatches"


def pin_dequant_golden():
    """Hand-packed rows decode to their hand-worked values, exactly."""
    for c in read_dequant_cases():
        N, K = c["N"], c["K"]
        q = np.array(cyc(c["bytes"], N * K // 2), dtype=np.uint8)
        sm = np.array(c["sm"], dtype=np.uint16)
        got = oracle.dequant(c["fmt"], q, sm, N, K).ravel()
        exp = np.array(cyc(c["expect"], N * K), dtype=np.float64)
        assert np.array_equal(got.astype(np.float64), exp), c["name"]


def pin_e4m3_decode_all():
    """Every E4M3 pattern against torch's float8_e4m3fn decoding (NaN where it is NaN)."""
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_value(b) for b in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def pin_dequant_fp8_golden():
    for c in read_dequant_fp8_cases():
        N, K = c["N"], c["K"]
        nb, kb = N // 128, K // 128
        q = np.array(cyc(c["bytes"], N * K), dtype=np.uint8).reshape(N, K)
        s = np.array(c["scale"], dtype=np.float32)
        assert s.size == nb * kb == len(c["expect"]), c["name"]
        got = oracle.dequant(oracle.FMT_FP8_B128, q, s, N, K).astype(np.float64)
        for bi, e in enumerate(c["expect"]):
            r, cc = divmod(bi, kb)
            blk = got[128 * r:128 * (r + 1), 128 * cc:128 * (cc + 1)].ravel()
            assert np.array_equal(blk, np.array(cyc(e, 128 * 128))), (c["name"], bi)


def pin_dequant_nvfp4_golden():
    for c in read_dequant_nvfp4_cases():
        N, K = c["N"], c["K"]
        q = np.array(cyc(c["bytes"], N * K // 2), dtype=np.uint8).reshape(N, K // 2)
        sb = np.array(c["scale"], dtype=np.uint8)
        assert sb.size == N * (K // 16) == len(c["expect"]), c["name"]
        got = oracle.dequant(oracle.FMT_NVFP4, q, sb, N, K, c["global"]).astype(np.float64)
        exp = np.concatenate([cyc(e, 16) for e in c["expect"]]).reshape(N, K)
        assert np.array_equal(got, exp), c["name"]


def pin_e2m1_table():
    """The 16 E2M1 codes: the hand-listed magnitudes, sign bit 3."""
    got = np.array([oracle.e2m1_value(c) for c in range(16)])
    assert np.array_equal(got, E2M1_TABLE)
    assert np.array_equal(np.signbit(got), np.arange(16) >= 8)


def pin_dequant_random():
    """Random rows: float32 of the exact value, as computed independently by numpy."""
    rng = np.random.default_rng(11)
    for fmt in (oracle.FMT_ASYM_G64, oracle.FMT_SYM_G128):
        N, K = 7, 384
        g = 64 if fmt == oracle.FMT_ASYM_G64 else 128
        q = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        ng = N * (K // g) * (2 if fmt == oracle.FMT_ASYM_G64 else 1)
        sm = rng.integers(0, 0x7c00, size=ng, dtype=np.uint16)
        sm |= (rng.integers(0, 2, size=ng, dtype=np.uint16) << 15)
        ref = np_dequant64(fmt, q, sm, N, K).astype(np.float32)
        got = oracle.dequant(fmt, q, sm, N, K)
        assert np.array_equal(got, ref)
    # fp8: every code with random float32 block scales (four blocks)
    N = K = 256
    q = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] -= 1
    sm = (rng.standard_normal((2, 2)) * 1e-3).astype(np.float32)
    ref = np_dequant64(oracle.FMT_FP8_B128, q, sm, N, K).astype(np.float32)
    got = oracle.dequant(oracle.FMT_FP8_B128, q, sm, N, K)
    assert np.array_equal(got, ref)
    # nvfp4: every code and block scale byte (no NaN), a global scale
    N, K = 5, 256
    q = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    sb = rng.integers(0, 256, size=(N, K // 16), dtype=np.uint8)
    sb[(sb & 0x7F) == 0x7F] -= 1
    ref = np_nvfp4_64(q, sb, 0.375, N, K).astype(np.float32)
    got = oracle.dequant(oracle.FMT_NVFP4, q, sb, N, K, 0.375)
    assert np.array_equal(got, ref)


def pin_router():
    """Logits = bf16 of the float64 product computed by numpy (plus bias), bit for bit."""
    rng = np.random.default_rng(3)
    for (T, H, E) in ((5, 256, 16), (3, 2048, 64)):
        x = rand_bf16(rng, (T, H))
        wr = rand_bf16(rng, (E, H), 0.02)
        bias = (rng.standard_normal(E) * 0.5).astype(np.float32)
        for b in (None, bias):
            acc = bf16_to_f64(x) @ bf16_to_f64(wr).T
            if b is not None:
                acc = acc + b.astype(np.float64)
            ref = torch_bf16_bits(acc.astype(np.float32))
            got = oracle.router(x, wr, T, H, E, b)
            assert np.array_equal(got, ref.reshape(T, E))


def _bf16_small_ints(rng, shape, hi):
    return torch_bf16_bits(rng.integers(-hi, hi + 1, size=shape).astype(np.float32) * 0.25)


def pin_topk_bruteforce():
    """Top-k = first k of a full stable sort by (logit descending, expert ascending)."""
    rng = np.random.default_rng(5)
    for (T, E, k) in ((64, 16, 2), (64, 256, 8), (16, 9, 9), (8, 5, 1)):
        for lg in (rand_bf16(rng, (T, E)), _bf16_small_ints(rng, (T, E), 3)):
            idx, _ = oracle.topk(lg, T, E, k)
            v = bf16_to_f64(lg).reshape(T, E)
            for t in range(T):
                order = np.lexsort((np.arange(E), -v[t]))
                assert list(idx[t]) == list(order[:k]), (T, E, k, t)


def pin_topk_adversarial():
    """All-equal logits give 0..k-1; ties straddling rank k go to the lower index; NaN ranks last."""
    E, k = 256, 8
    lg = np.full((1, E), torch_bf16_bits(np.float32([0.5]))[0], dtype=np.uint16)
    idx, gate = oracle.topk(lg, 1, E, k)
    assert list(idx[0]) == list(range(k))
    assert np.allclose(gate, 1.0 / k, rtol=1e-7, atol=0)
    vals = np.zeros(E, dtype=np.float32)
    vals[[200, 100, 50, 3]] = 2.0          # four leaders
    vals[[250, 9, 180, 77, 8, 130]] = 1.0  # six tied for the last four places
    lg = torch_bf16_bits(vals)[None, :]
    idx, _ = oracle.topk(lg, 1, E, k)
    assert list(idx[0]) == [3, 50, 100, 200, 8, 9, 77, 130]
    vals = np.zeros(E, dtype=np.float32)
    vals[:k] = np.nan
    lg = torch_bf16_bits(vals)[None, :]
    idx, _ = oracle.topk(lg, 1, E, k)
    assert list(idx[0]) == list(range(k, 2 * k))


def pin_topk_signed_zero_and_nan():
    """-0 equals +0 and a NaN ranks as -inf: both are ties that go to the lower
    expert index (the plain ordering of values, NaN read as -inf).  The
    expected indices are written out by hand; the selected NaN / -inf slot
    has gate exactly 0."""
    E, k = 16, 4
    bits = np.full(E, 0xbf80, dtype=np.uint16)     # -1.0 everywhere
    bits[[9, 2, 14]] = [0x4000, 0x3f80, 0x3f00]      # 2.0, 1.0, 0.5: three leaders
    bits[[5, 7, 11]] = [0x8000, 0x0000, 0x8000]      # -0 at 5, +0 at 7, -0 at 11
    idx, gate = oracle.topk(bits[None, :], 1, E, k)
    assert list(idx[0]) == [9, 2, 14, 5], idx
    bits[5] = 0x0000                                 # +0 at 5, -0 at 11: still 5
    bits[3] = 0x8000                                 # -0 at 3 comes first now
    idx, _ = oracle.topk(bits[None, :], 1, E, k)
    assert list(idx[0]) == [9, 2, 14, 3], idx
    bits = np.full(E, 0xff80, dtype=np.uint16)     # -inf everywhere
    bits[[0, 6]] = [0x7fc0, 0xffc1]                  # quiet NaN at 0, negative NaN at 6
    bits[[12, 4, 8]] = [0x3f80, 0x3f80, 0xc000]      # 1.0, 1.0, -2.0
    idx, gate = oracle.topk(bits[None, :], 1, E, k)
    assert list(idx[0]) == [4, 12, 8, 0], idx        # NaN at 0 ties the -inf run, lowest index
    assert gate[0, 3] == 0.0 and gate[0, 0] == gate[0, 1] > 0
    idx, _ = oracle.topk(bits[None, :], 1, E, 6)
    assert list(idx[0]) == [4, 12, 8, 0, 1, 2], idx


def pin_gates():
    """Gates: softmax over all experts renormalised over the selected; sums; special cases."""
    rng = np.random.default_rng(9)
    for (T, E, k) in ((32, 256, 8), (32, 16, 2), (8, 12, 12), (8, 40, 1)):
        lg = rand_bf16(rng, (T, E), 1.5)
        idx, gate = oracle.topk(lg, T, E, k)
        v = bf16_to_f64(lg).reshape(T, E)
        full = scipy.special.softmax(v, axis=1)
        for t in range(T):
            sel = full[t, idx[t]]
            ref = sel / sel.sum()
            assert np.allclose(gate[t], ref, rtol=1e-6, atol=0)
            assert abs(float(gate[t].astype(np.float64).sum()) - 1.0) <= 1e-6
            if k == 1:
                assert gate[t, 0] == 1.0
            if k == E:
                assert np.allclose(gate[t], full[t, idx[t]], rtol=1e-6, atol=0)


def pin_group():
    """Grouping = numpy's stable argsort of the flat expert ids; offsets and inverse consistent."""
    rng = np.random.default_rng(13)
    for (T, k, E) in ((1, 8, 256), (37, 2, 16), (512, 8, 256), (64, 4, 5)):
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        cnt, off, perm, inv = oracle.group(idx, T, k, E)
        flat = idx.ravel()
        assert np.array_equal(cnt, np.bincount(flat, minlength=E))
        assert off[0] == 0 and off[E] == T * k and np.all(np.diff(off) == cnt)
        assert np.array_equal(perm, np.argsort(flat, kind="stable"))
        assert np.array_equal(inv[perm], np.arange(T * k))
        assert np.array_equal(np.sort(perm), np.arange(T * k))


def pin_one_expert_dense():
    """E = 1, k = 1: the layer is the dense SwiGLU MLP of the dequantised weights."""
    rng = np.random.default_rng(17)
    for fmt, (H, I) in ((oracle.FMT_ASYM_G64, (128, 64)), (oracle.FMT_SYM_G128, (256, 128)),
                        (oracle.FMT_FP8_B128, (256, 128)), (oracle.FMT_NVFP4, (128, 64))):
        T = 3
        mats = rand_layer(rng, 1, H, I, fmt)
        x = rand_bf16(rng, (T, H))
        idx = np.zeros((T, 1), dtype=np.int32)
        gate = np.ones((T, 1), dtype=np.float32)
        y = oracle.experts(fmt, 1, H, I, *layer_args(mats), x, idx, gate, T, 1, **glob_kw(mats))
        for t in range(T):
            ref = np_expert_out(fmt, mats, 0, bf16_to_f64(x[t]), H, I)
            assert rel_l2(y[t], ref) < 1e-6
            assert np.allclose(y[t], ref, rtol=1e-6, atol=1e-6)


def pin_experts_bruteforce():
    """Several experts, top-k routing, gate-weighted sum: float64 numpy per token."""
    rng = np.random.default_rng(19)
    for fmt, (E, H, I, k, T) in ((oracle.FMT_ASYM_G64, (6, 128, 64, 3, 5)),
                                 (oracle.FMT_SYM_G128, (5, 256, 128, 2, 4)),
                                 (oracle.FMT_FP8_B128, (3, 256, 128, 2, 3)),
                                 (oracle.FMT_NVFP4, (4, 128, 64, 2, 4))):
        mats = rand_layer(rng, E, H, I, fmt)
        x = rand_bf16(rng, (T, H))
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        gate = rng.random((T, k)).astype(np.float32)
        y = oracle.experts(fmt, E, H, I, *layer_args(mats), x, idx, gate, T, k, **glob_kw(mats))
        for t in range(T):
            ref = sum(float(gate[t, i]) * np_expert_out(fmt, mats, idx[t, i], bf16_to_f64(x[t]), H, I)
                      for i in range(k))
            assert rel_l2(y[t], ref) < 1e-6
        sub = [4, 1] if T > 4 else [1]
        ys = oracle.experts(fmt, E, H, I, *layer_args(mats), x, idx, gate, T, k, tokens=sub, **glob_kw(mats))
        assert np.array_equal(ys, y[sub])


def pin_gate_linearity():
    """Two byte-identical experts selected together give the single expert's output."""
    rng = np.random.default_rng(23)
    fmt, H, I, T = oracle.FMT_ASYM_G64, 128, 64, 4
    one = rand_layer(rng, 1, H, I, fmt)
    two = {n: np.concatenate([a, a]) for n, a in one.items()}
    x = rand_bf16(rng, (T, H))
    lg = torch_bf16_bits(np.tile(np.float32([[0.25, -0.75]]), (T, 1)))
    idx2, gate2 = oracle.topk(lg, T, 2, 2)
    assert np.all(np.sort(idx2, axis=1) == [0, 1])
    y2 = oracle.experts(fmt, 2, H, I, *layer_args(two), x, idx2, gate2, T, 2)
    y1 = oracle.experts(fmt, 1, H, I, *layer_args(one), x, np.zeros((T, 1), np.int32),
                        np.ones((T, 1), np.float32), T, 1)
    assert rel_l2(y2, y1) < 1e-6


def pin_layer_chain():
    """Router + top-k + experts composed through moe_layer agree with the pieces."""
    rng = np.random.default_rng(29)
    fmt, E, H, I, k, T = oracle.FMT_ASYM_G64, 8, 128, 64, 2, 6
    mats = rand_layer(rng, E, H, I, fmt)
    x = rand_bf16(rng, (T, H))
    wr = rand_bf16(rng, (E, H), 0.05)
    lg = oracle.router(x, wr, T, H, E)
    idx, gate = oracle.topk(lg, T, E, k)
    y = oracle.experts(fmt, E, H, I, *layer_args(mats), x, idx, gate, T, k)
    v = bf16_to_f64(lg).reshape(T, E)
    for t in range(T):
        sel = np.lexsort((np.arange(E), -v[t]))[:k]
        w = scipy.special.softmax(v[t, sel])
        ref = sum(w[i] * np_expert_out(fmt, mats, sel[i], bf16_to_f64(x[t]), H, I) for i in range(k))
        assert rel_l2(y[t], ref) < 1e-6


def pin_residual():
    """x' = bf16(float32(x) + y) matches torch's float32 add and bf16 rounding."""
    rng = np.random.default_rng(31)
    x = rand_bf16(rng, (4, 300))
    y = (rng.standard_normal((4, 300)) * 0.3).astype(np.float32)
    got = oracle.residual(x, y)
    xt = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).float()
    ref = (xt + torch.from_numpy(y)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def pin_dequant_int8_golden():
    for c in read_dequant_int8_cases():
        N, K = c["N"], c["K"]
        q = np.array(cyc(c["bytes"], N * K), dtype=np.uint8).view(np.int8).reshape(N, K)
        s = np.array(c["scale"], dtype=np.uint16)
        assert s.size == N * (K // 128) == len(c["expect"]), c["name"]
        exp = np.concatenate([cyc(e, 128) for e in c["expect"]]).reshape(N, K)
        got = oracle.dequant_int8(q, s, N, K)
        assert np.array_equal(got.astype(np.float64), exp), c["name"]


def pin_dequant_int8_random():
    rng = np.random.default_rng(37)
    for N, K in ((3, 128), (5, 384), (2, 2048)):
        q = rng.integers(-128, 128, size=(N, K)).astype(np.int8)
        s = rng.integers(0, 0x7c00, size=(N, K // 128)).astype(np.uint16)
        s[0, 0] |= 0x8000  # a negative scale
        got = oracle.dequant_int8(q, s, N, K)
        assert np.array_equal(got, np_dequant_int8_64(q, s, N, K).astype(np.float32))


def pin_shared_dense():
    """The shared expert against float64 numpy, with and without y_in, on all
    tokens and on a subset."""
    rng = np.random.default_rng(41)
    for H, I, T in ((128, 128, 3), (256, 384, 5)):
        mats = rand_shared(rng, H, I)
        x = rand_bf16(rng, (T, H))
        y = oracle.shared(H, I, *shared_args(mats), x, T)
        ref = np.stack([np_shared_out(mats, bf16_to_f64(x[t]), H, I) for t in range(T)])
        assert rel_l2(y, ref) < 1e-6
        assert np.allclose(y, ref, rtol=1e-6, atol=1e-7)
        sub = [T - 1, 0]
        y_in = rng.standard_normal((2, H)).astype(np.float32)
        ys = oracle.shared(H, I, *shared_args(mats), x, T, tokens=sub, y_in=y_in)
        assert np.allclose(ys, ref[sub] + y_in.astype(np.float64), rtol=1e-6, atol=1e-6)


def pin_shared_as_routed_expert():
    """Codes within [-8, 7] make the shared expert a sym-g128 int4 expert: the
    routed one-expert top-1 layer of the same weights gives the same output."""
    rng = np.random.default_rng(43)
    H, I, T = 256, 128, 4
    mats = rand_shared(rng, H, I, -8, 7)
    routed = {}
    for name in ("gate", "up", "down"):
        q = mats[name + "_q"].astype(np.int64) + 8
        routed[name + "_q"] = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)[None]
        routed[name + "_sm"] = mats[name + "_s"][None]
    x = rand_bf16(rng, (T, H))
    y1 = oracle.experts(oracle.FMT_SYM_G128, 1, H, I, *layer_args(routed), x, np.zeros((T, 1), np.int32),
                        np.ones((T, 1), np.float32), T, 1)
    ys = oracle.shared(H, I, *shared_args(mats), x, T)
    assert rel_l2(ys, y1) < 1e-12


ALL_PINS = [pin_f16_decode_all, pin_bf16_decode_all, pin_bf16_round, pin_dequant_golden,
            pin_dequant_random, pin_router, pin_topk_bruteforce, pin_topk_adversarial, pin_topk_signed_zero_and_nan,
            pin_gates, pin_group, pin_one_expert_dense, pin_experts_bruteforce,
            pin_gate_linearity, pin_layer_chain, pin_residual, pin_dequant_int8_golden,
            pin_dequant_int8_random, pin_shared_dense, pin_shared_as_routed_expert, pin_e4m3_decode_all,
            pin_dequant_fp8_golden, pin_e2m1_table, pin_dequant_nvfp4_golden]
