"""Seeded synthetic inputs for the routed int4 MoE expert layer.

This module is shared by the tests, the benchmark and the oracle's callers.  It
draws random tensors and encodes expert weights into the two int4 group
formats; it holds none of the layer's own arithmetic (no router product, no
top-k, no grouping, no expert MLP, no combine).

Sources of the recipe (drama-rs / drama-q4 / drama-3-w4a16 model pages):
  * expert weights are int4 with a per-group f16 scale and f16 min, group 64
    along the input dimension (drama-q4 card, "What's quantized" table), or
    int4 symmetric with one f16 scale per 128 input weights
    (drama-3-w4a16 card, "At a glance" table and "How it was made");
  * each scale is picked from 20 clipping ratios 1.0 down to 0.81 by least
    squared error, with no calibration data (drama-3-w4a16, "How it was
    made"; drama-q4 names the same "MSE clip search");
  * router, activations: bf16 (drama-q4 "What's quantized": router bf16);
  * block-FP8 experts: E4M3 codes with one float32 scale per block of 128
    rows x 128 inputs, the released experts' format (drama-3-w4a16 card,
    "At a glance": routed experts block-FP8 with 128 x 128 scales; "How it
    was made": each matrix dequantised with its block scales);
  * NVFP4 experts: packed E2M1 values, one E4M3 scale per 16 input weights
    and a float32 global scale per matrix, gate and up sharing theirs within
    an expert, converted by round-to-nearest (drama-3-nvfp4 card,
    "Quantization").

Random streams: every tensor gets its own torch.Generator seeded from
(config seed, tensor tag) through a fixed 64-bit mix, so tensors do not depend
on the order they are drawn in.  Generation runs on the device that will hold
the tensor (torch's CPU and GPU generators differ, so the same seed gives
different values on the two; each test draws on one device only).

Layout written here (the library's canonical layout):
  packed nibbles  uint8  [E][N][K/2], byte j of a row holds k = 2j in its low
                  nibble and k = 2j+1 in its high nibble;
  asym scale/min  uint16 (f16 bits) [E][N][K/64][2] = {scale, min};
  sym scale       uint16 (f16 bits) [E][N][K/128];
  fp8 codes       uint8 (E4M3 bits) [E][N][K], one byte per weight;
  fp8 scale       float32 [E][N/128][K/128];
  nvfp4 codes     uint8 [E][N][K/2], E2M1 nibbles packed as the int4 codes;
  nvfp4 scale     uint8 (E4M3 bits) [E][N][K/16]; global float32 [E][2] =
                  {gate and up, down};
  gate, up: N = inter, K = hidden; down: N = hidden, K = inter.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import torch

FMT_ASYM_G64 = 0
FMT_SYM_G128 = 1
FMT_FP8_B128 = 2
FMT_NVFP4 = 3
GROUP = {FMT_ASYM_G64: 64, FMT_SYM_G128: 128, FMT_FP8_B128: 128, FMT_NVFP4: 16}
E4M3_MAX = 448.0
# magnitudes of the 4-bit float E2M1 for codes 0..7 (bit 3 is the sign)
E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)

# 20 clipping ratios, 1.00, 0.99, ..., 0.81 (drama-3-w4a16, "How it was made").
CLIP_RATIOS = tuple(round(1.0 - 0.01 * i, 2) for i in range(20))

# Rows quantised per chunk, to bound temporaries on the host.
_CHUNK_ELEMS = 1 << 24


def stream_seed(seed: int, tag: str) -> int:
    """64-bit seed for the tensor named ``tag`` under config seed ``seed``."""
    h = hashlib.blake2b(f"{seed}:{tag}".encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def generator(seed: int, tag: str, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(stream_seed(seed, tag))
    return g


def normal(shape, std: float, seed: int, tag: str, device="cpu") -> torch.Tensor:
    """float32 N(0, std^2) of ``shape``."""
    g = generator(seed, tag, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def bf16_bits(t: torch.Tensor) -> torch.Tensor:
    """Round float32 to bf16 (round-to-nearest-even) and return the raw bits as int16."""
    return t.to(torch.bfloat16).view(torch.int16)


def f16_bits(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.float16).view(torch.int16)


def pack_nibbles(q: torch.Tensor) -> torch.Tensor:
    """q: uint8 [..., K] with values 0..15 -> uint8 [..., K/2] (even k in the low nibble)."""
    q = q.to(torch.uint8)
    lo = q[..., 0::2]
    hi = q[..., 1::2]
    return (lo | (hi << 4)).contiguous()


def _quantize_asym_rows(w: torch.Tensor, g: int, ratios):
    """w: float32 [R, K] -> (q uint8 [R, K], scale f16 [R, K/g], min f16 [R, K/g])."""
    R, K = w.shape
    wg = w.reshape(R, K // g, g)
    wmin = wg.amin(dim=2)
    wmax = wg.amax(dim=2)
    best_err = None
    best_q = best_s = best_m = None
    for r in ratios:
        lo = (wmin * r).to(torch.float16)
        s16 = ((wmax * r - wmin * r) / 15.0).to(torch.float16)
        m = lo.float().unsqueeze(2)
        s = s16.float().unsqueeze(2)
        safe = torch.where(s > 0, s, torch.ones_like(s))
        q = torch.round((wg - m) / safe).clamp_(0, 15)
        q = torch.where(s > 0, q, torch.zeros_like(q))
        err = ((q * s + m) - wg).square_().sum(dim=2)
        if best_err is None:
            best_err, best_q, best_s, best_m = err, q, s16, lo
        else:
            better = err < best_err  # ties keep the earlier (larger) ratio
            best_err = torch.where(better, err, best_err)
            best_q = torch.where(better.unsqueeze(2), q, best_q)
            best_s = torch.where(better, s16, best_s)
            best_m = torch.where(better, lo, best_m)
    return best_q.reshape(R, K).to(torch.uint8), best_s, best_m


def _quantize_sym_rows(w: torch.Tensor, g: int, ratios):
    """w: float32 [R, K] -> (stored code q+8 uint8 [R, K], scale f16 [R, K/g])."""
    R, K = w.shape
    wg = w.reshape(R, K // g, g)
    amax = wg.abs().amax(dim=2)
    best_err = None
    best_q = best_s = None
    for r in ratios:
        s16 = (amax * r / 7.0).to(torch.float16)
        s = s16.float().unsqueeze(2)
        safe = torch.where(s > 0, s, torch.ones_like(s))
        q = torch.round(wg / safe).clamp_(-8, 7)
        q = torch.where(s > 0, q, torch.zeros_like(q))
        err = ((q * s) - wg).square_().sum(dim=2)
        if best_err is None:
            best_err, best_q, best_s = err, q, s16
        else:
            better = err < best_err
            best_err = torch.where(better, err, best_err)
            best_q = torch.where(better.unsqueeze(2), q, best_q)
            best_s = torch.where(better, s16, best_s)
    return (best_q + 8).reshape(R, K).to(torch.uint8), best_s


def quantize_fp8(w: torch.Tensor):
    """Encode float32 weights [..., N, K] as E4M3 with one float32 scale per
    128 x 128 block: scale = max |w| / 448 over the block, codes =
    e4m3(w / scale) (torch's round-to-nearest-even cast; an all-zero block
    gets scale 0 and codes 0).  Returns (codes uint8 [..., N, K], scales
    float32 [..., N/128, K/128])."""
    *lead, N, K = w.shape
    if N % 128 or K % 128:
        raise ValueError(f"({N}, {K}) is not a multiple of the 128 x 128 block")
    wb = w.reshape(-1, N // 128, 128, K // 128, 128).float()
    amax = wb.abs().amax(dim=(2, 4))
    sc = amax / E4M3_MAX
    safe = torch.where(sc > 0, sc, torch.ones_like(sc))[:, :, None, :, None]
    v = (wb / safe).clamp_(-E4M3_MAX, E4M3_MAX)
    q = v.to(torch.float8_e4m3fn).view(torch.uint8)
    return q.reshape(*lead, N, K).contiguous(), sc.reshape(*lead, N // 128, K // 128).contiguous()


def _e2m1_codes(v: torch.Tensor) -> torch.Tensor:
    """Nearest E2M1 code of each value (magnitudes above 6 saturate; ties go
    to the code with an even mantissa bit).  Returns uint8 codes 0..15."""
    grid = torch.tensor(E2M1_GRID, dtype=torch.float32, device=v.device)
    mids = (grid[1:] + grid[:-1]) / 2
    a = v.abs().clamp(max=6.0)
    idx = torch.bucketize(a, mids)  # mids[idx - 1] < a <= mids[idx]
    tie = (idx < 7) & (a == mids[idx.clamp(max=6)])
    idx = torch.where(tie & (idx % 2 == 1), idx + 1, idx)
    neg = (v < 0) & (idx > 0)
    return (idx + 8 * neg.to(idx.dtype)).to(torch.uint8)


def quantize_nvfp4(w: torch.Tensor, global_amax: torch.Tensor):
    """Encode float32 weights [B, N, K] as NVFP4 with the given per-matrix
    amax [B] that sets the global scale (the gate and up projections of an
    expert pass the larger of their two).

    global = amax / (6 * 448); each block of 16 inputs gets the E4M3 scale
    e4m3(block amax / (6 * global)) and codes e2m1(w / (scale * global)).
    Returns (packed uint8 [B, N, K/2], E4M3 scales uint8 [B, N, K/16],
    global float32 [B])."""
    B, N, K = w.shape
    g = global_amax.float() / (6.0 * E4M3_MAX)
    gs = torch.where(g > 0, g, torch.ones_like(g))[:, None, None]
    wb = w.float().reshape(B, N, K // 16, 16)
    sb = (wb.abs().amax(dim=3) / (6.0 * gs)).clamp_(max=E4M3_MAX).to(torch.float8_e4m3fn)
    den = sb.float() * gs
    v = torch.where(den[..., None] > 0, wb / torch.where(den > 0, den, torch.ones_like(den))[..., None],
                    torch.zeros_like(wb))
    codes = _e2m1_codes(v).reshape(B, N, K)
    return pack_nibbles(codes), sb.view(torch.uint8).contiguous(), g.contiguous()


def quantize(w: torch.Tensor, fmt: int, clip: bool = True):
    """Encode float32 weights [..., N, K] (groups along K).

    Returns (packed uint8 [..., N, K/2], scale/min int16 bits):
      asym g64: [..., N, K/64, 2] = {scale, min};  sym g128: [..., N, K/128];
    fp8 b128: (codes uint8 [..., N, K], float32 scales [..., N/128, K/128]).
    ``clip`` selects the 20-ratio least-squares search; without it only r = 1
    (plain round-to-nearest) is used.
    """
    if fmt == FMT_FP8_B128:
        return quantize_fp8(w)
    g = GROUP[fmt]
    *lead, N, K = w.shape
    if K % g:
        raise ValueError(f"K={K} is not a multiple of the group {g}")
    ratios = CLIP_RATIOS if clip else (1.0,)
    rows = w.reshape(-1, K)
    R = rows.shape[0]
    step = max(1, _CHUNK_ELEMS // K) if rows.device.type == "cpu" else max(1, (1 << 27) // K)
    packed = torch.empty((R, K // 2), dtype=torch.uint8, device=w.device)
    if fmt == FMT_ASYM_G64:
        sm = torch.empty((R, K // g, 2), dtype=torch.int16, device=w.device)
    else:
        sm = torch.empty((R, K // g), dtype=torch.int16, device=w.device)
    for r0 in range(0, R, step):
        r1 = min(R, r0 + step)
        chunk = rows[r0:r1].float()
        if fmt == FMT_ASYM_G64:
            q, s, m = _quantize_asym_rows(chunk, g, ratios)
            sm[r0:r1, :, 0] = s.view(torch.int16)
            sm[r0:r1, :, 1] = m.view(torch.int16)
        else:
            q, s = _quantize_sym_rows(chunk, g, ratios)
            sm[r0:r1] = s.view(torch.int16)
        packed[r0:r1] = pack_nibbles(q)
    return packed.reshape(*lead, N, K // 2), sm.reshape(*lead, N, *sm.shape[1:])


@dataclasses.dataclass
class Layer:
    """One MoE layer's routed experts in the canonical packed layout."""
    fmt: int
    num_experts: int
    hidden: int
    inter: int
    gate_q: torch.Tensor
    up_q: torch.Tensor
    down_q: torch.Tensor
    gate_sm: torch.Tensor
    up_sm: torch.Tensor
    down_sm: torch.Tensor
    global_scale: torch.Tensor | None = None  # NVFP4: float32 [E][2] = {gate and up, down}

    @property
    def group(self) -> int:
        return GROUP[self.fmt]

    def to(self, device) -> "Layer":
        kw = {f.name: getattr(self, f.name) for f in dataclasses.fields(self)}
        for k, v in kw.items():
            if isinstance(v, torch.Tensor):
                kw[k] = v.to(device)
        return Layer(**kw)

    def tensors(self):
        return (self.gate_q, self.up_q, self.down_q, self.gate_sm, self.up_sm, self.down_sm)

    def nbytes(self) -> int:
        extra = self.global_scale.numel() * 4 if self.global_scale is not None else 0
        return sum(t.numel() * t.element_size() for t in self.tensors()) + extra

    def expert_nbytes(self) -> int:
        return self.nbytes() // self.num_experts


def make_layer(E: int, H: int, I: int, fmt: int, seed: int, tag: str = "layer",
               clip: bool = True, std: float = 0.02, device="cpu") -> Layer:
    """Draw N(0, std^2) float32 gate/up/down weights for E experts and encode them."""
    if fmt == FMT_NVFP4:
        return _make_layer_nvfp4(E, H, I, seed, tag, std, device)
    out = {}
    # experts are drawn from their own streams, then encoded a batch at a time
    batch = max(1, (1 << 26) // (H * I)) if torch.device(device).type == "cpu" else E
    for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        qs, sms = [], []
        for e0 in range(0, E, batch):
            e1 = min(E, e0 + batch)
            w = torch.empty((e1 - e0, N, K), dtype=torch.float32, device=device)
            for e in range(e0, e1):
                w[e - e0] = normal((N, K), std, seed, f"{tag}/{name}/{e}", device)
            q, sm = quantize(w, fmt, clip)
            qs.append(q)
            sms.append(sm)
            del w
        out[name + "_q"] = torch.cat(qs).contiguous()
        out[name + "_sm"] = torch.cat(sms).contiguous()
    return Layer(fmt=fmt, num_experts=E, hidden=H, inter=I, **out)


def _make_layer_nvfp4(E, H, I, seed, tag, std, device) -> Layer:
    """make_layer for NVFP4: the gate and up projections of an expert share
    one global scale (the larger amax of the two)."""
    out = {n: [] for n in ("gate_q", "up_q", "down_q", "gate_sm", "up_sm", "down_sm")}
    glob = []
    batch = max(1, (1 << 26) // (H * I)) if torch.device(device).type == "cpu" else 64
    for e0 in range(0, E, batch):
        e1 = min(E, e0 + batch)
        mats = {}
        for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            mats[name] = torch.stack([normal((N, K), std, seed, f"{tag}/{name}/{e}", device) for e in range(e0, e1)])
        amax = lambda t: t.abs().flatten(1).amax(dim=1)
        gu = torch.maximum(amax(mats["gate"]), amax(mats["up"]))
        gl = []
        for name, ga in (("gate", gu), ("up", gu), ("down", amax(mats["down"]))):
            q, sb, g = quantize_nvfp4(mats[name], ga)
            out[name + "_q"].append(q)
            out[name + "_sm"].append(sb)
            gl.append(g)
        glob.append(torch.stack([gl[0], gl[2]], dim=1))
        del mats
    kw = {n: torch.cat(v).contiguous() for n, v in out.items()}
    return Layer(fmt=FMT_NVFP4, num_experts=E, hidden=H, inter=I, global_scale=torch.cat(glob).contiguous(), **kw)


def zipf_logits(T: int, E: int, s: float, seed: int, device="cpu") -> torch.Tensor:
    """bf16 bits [T][E]: ln p_{pi(e)} + Gumbel(0,1), p_r proportional to r^-s.

    Taking the top-k of Gumbel-perturbed log-probabilities draws k experts
    without replacement with probabilities proportional to p, so expert
    popularity follows the Zipf law over a seeded permutation pi of the experts.
    """
    g = generator(seed, "zipf/perm", device)
    perm = torch.randperm(E, generator=g, device=device)
    ranks = torch.arange(1, E + 1, device=device, dtype=torch.float64)
    p = ranks.pow(-s)
    p = p / p.sum()
    logp = torch.log(p)[perm].float()  # expert e gets rank perm[e]
    g2 = generator(seed, "zipf/gumbel", device)
    u = torch.rand((T, E), generator=g2, device=device, dtype=torch.float64)
    u = u.clamp_(min=1e-300)
    gumbel = -torch.log(-torch.log(u))
    return bf16_bits((logp.unsqueeze(0).double() + gumbel).float())


# ------------------------------------------------------------ shared expert

INT8_GROUP = 128


def quantize_int8(w: torch.Tensor):
    """Encode float32 weights [..., N, K] as int8 symmetric group 128 along K.

    The shared expert's linears use this format (drama-q4 card, "What's
    quantized": int8, symmetric, group 128).  Each group's f16 scale is
    f16(max |w| / 127) and q = clamp(round(w / scale), -127, 127); an all-zero
    group gets scale 0 and codes 0.  Returns (q int8 [..., N, K], scale int16
    bits [..., N, K/128]).
    """
    *lead, N, K = w.shape
    if K % INT8_GROUP:
        raise ValueError(f"K={K} is not a multiple of {INT8_GROUP}")
    wg = w.reshape(-1, K // INT8_GROUP, INT8_GROUP).float()
    s16 = (wg.abs().amax(dim=2) / 127.0).to(torch.float16)
    s = s16.float().unsqueeze(2)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    q = torch.round(wg / safe).clamp_(-127, 127)
    q = torch.where(s > 0, q, torch.zeros_like(q))
    return (q.to(torch.int8).reshape(*lead, N, K).contiguous(),
            s16.view(torch.int16).reshape(*lead, N, K // INT8_GROUP).contiguous())


@dataclasses.dataclass
class SharedExpert:
    """A layer's shared expert (SwiGLU MLP every token passes through), int8
    symmetric group 128: q int8 [N][K], scale f16 bits [N][K/128];
    gate, up: (N, K) = (inter, hidden); down: (hidden, inter)."""
    hidden: int
    inter: int
    gate_q: torch.Tensor
    up_q: torch.Tensor
    down_q: torch.Tensor
    gate_s: torch.Tensor
    up_s: torch.Tensor
    down_s: torch.Tensor

    def to(self, device) -> "SharedExpert":
        kw = {f.name: getattr(self, f.name) for f in dataclasses.fields(self)}
        for k, v in kw.items():
            if isinstance(v, torch.Tensor):
                kw[k] = v.to(device)
        return SharedExpert(**kw)

    def tensors(self):
        return (self.gate_q, self.up_q, self.down_q, self.gate_s, self.up_s, self.down_s)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.tensors())


def make_shared(H: int, I: int, seed: int, tag: str = "shared", std: float = 0.02,
                device="cpu") -> SharedExpert:
    """Draw N(0, std^2) gate/up/down weights of a shared expert and encode them."""
    out = {}
    for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        q, s = quantize_int8(normal((N, K), std, seed, f"{tag}/{name}", device))
        out[name + "_q"] = q
        out[name + "_s"] = s
    return SharedExpert(hidden=H, inter=I, **out)


def random_shared(H: int, I: int, seed: int, device="cpu", tag="rand_shared") -> SharedExpert:
    """Shared expert with uniformly random codes in [-127, 127] and scales
    around the N(0, 0.02) statistics (1.2e-4 .. 2.4e-4), for shape tests."""
    out = {}
    for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        gen = generator(seed, f"{tag}/{name}", device)
        q = torch.randint(-127, 128, (N, K), generator=gen, device=device, dtype=torch.int32)
        out[name + "_q"] = q.to(torch.int8)
        s = torch.rand((N, K // INT8_GROUP), generator=gen, device=device) * 1.2e-4 + 1.2e-4
        out[name + "_s"] = f16_bits(s).contiguous()
    return SharedExpert(hidden=H, inter=I, **out)


@dataclasses.dataclass
class Case:
    """A complete set of inputs for one MoE layer call (or a chain of layers)."""
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    fmt: int
    x: torch.Tensor            # int16 bf16 bits [T][H]
    router_w: torch.Tensor | None   # int16 bf16 bits [E][H] (None when logits are given)
    logits: torch.Tensor | None     # int16 bf16 bits [T][E] when given directly
    layers: list               # list[Layer] (one per layer)
    router_ws: list | None = None   # per-layer router weights for chains


CONFIGS = {
    # name: (T, H, E, k, I, fmt, clip, router)
    1: ("tiny", 4, 256, 16, 2, 128, FMT_ASYM_G64, False, "gemv"),
    2: ("decode", 1, 2048, 256, 8, 512, FMT_ASYM_G64, True, "gemv"),
    3: ("prefill_zipf", 512, 2048, 256, 8, 512, FMT_ASYM_G64, True, "zipf"),
    4: ("frame", 16, 2048, 256, 8, 512, FMT_ASYM_G64, False, "gemv"),
    5: ("long_prefill_sym", 4096, 2048, 256, 8, 512, FMT_SYM_G128, True, "normal"),
}
FRAME_LAYERS = 40


def make_case(cfg: int, device="cpu", seed: int = 0, layers: int | None = None,
              T: int | None = None, fmt: int | None = None) -> Case:
    """Inputs of one of the five workload configurations (seed 0 by default).

    ``layers`` overrides the 40-layer depth of the frame configuration and
    ``T`` the token count (both for smaller runs of the same recipe); ``fmt``
    encodes the same Gaussian weights in another expert format (e.g. block
    FP8, the released experts' format).
    """
    name, T0, H, E, k, I, fmt0, clip, router = CONFIGS[cfg]
    fmt = fmt0 if fmt is None else fmt
    T = T0 if T is None else T
    nl = (FRAME_LAYERS if layers is None else layers) if cfg == 4 else 1
    x = bf16_bits(normal((T, H), 1.0, seed, f"{name}/x", device))
    lay, rws = [], []
    for l in range(nl):
        # configs 2 and 3 share one set of expert weights
        wtag = "shared_2_3" if cfg in (2, 3) else f"{name}/L{l}"
        lay.append(make_layer(E, H, I, fmt, seed, wtag, clip=clip, device=device))
        if router == "gemv":
            rtag = "shared_2_3/router" if cfg in (2, 3) else f"{name}/L{l}/router"
            rws.append(bf16_bits(normal((E, H), 0.02, seed, rtag, device)))
    logits = None
    if router == "zipf":
        logits = zipf_logits(T, E, 1.1, seed, device)
    elif router == "normal":
        logits = bf16_bits(normal((T, E), 1.0, seed, f"{name}/logits", device))
    return Case(name=name, T=T, H=H, E=E, k=k, I=I, fmt=fmt, x=x,
                router_w=rws[0] if rws else None, logits=logits, layers=lay,
                router_ws=rws if rws else None)


def _log2_uniform(shape, lo, hi, gen, device):
    """2^u with u uniform in [lo, hi)."""
    return torch.exp2(torch.rand(shape, generator=gen, device=device) * (hi - lo) + lo)


def random_layer(E, H, I, fmt, seed, device="cpu", tag="rand", log2_scale=None) -> Layer:
    """Layer with uniformly random codes and scales drawn around the N(0, 0.02) statistics.

    Used for shapes where the clip search would be slow and only the byte
    layout matters (tests of the kernels' indexing at odd shapes).  With
    log2_scale = (lo, hi) the scales are drawn log-uniformly from [2^lo, 2^hi)
    instead (int4 group scales, the asymmetric min at -6 to -9 scales;
    block-FP8 block scales; NVFP4 global scales, with E4M3 block scales
    over their whole positive range), for tests of the numerics at extreme
    magnitudes.
    """
    g = GROUP[fmt]
    out = {}
    if fmt == FMT_NVFP4 and log2_scale is not None:
        for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            gen = generator(seed, f"{tag}/{name}", device)
            q = torch.randint(0, 256, (E, N, K // 2), generator=gen, device=device, dtype=torch.int32)
            out[name + "_q"] = q.to(torch.uint8)
            # every finite positive E4M3 scale (0x01 .. 0x7e, 2^-9 .. 448)
            sb = torch.randint(0x01, 0x7f, (E, N, K // 16), generator=gen, device=device, dtype=torch.int32)
            out[name + "_sm"] = sb.to(torch.uint8)
        gen = generator(seed, f"{tag}/global", device)
        glob = _log2_uniform((E, 2), log2_scale[0], log2_scale[1], gen, device)
        return Layer(fmt=fmt, num_experts=E, hidden=H, inter=I, global_scale=glob, **out)
    if fmt == FMT_FP8_B128 and log2_scale is not None:
        for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            gen = generator(seed, f"{tag}/{name}", device)
            q = torch.randint(0, 256, (E, N, K), generator=gen, device=device, dtype=torch.int32)
            q = torch.where((q & 0x7f) == 0x7f, q - 1, q)  # no NaN codes
            out[name + "_q"] = q.to(torch.uint8)
            out[name + "_sm"] = _log2_uniform((E, N // 128, K // 128), log2_scale[0], log2_scale[1], gen,
                                              device).contiguous()
        return Layer(fmt=fmt, num_experts=E, hidden=H, inter=I, **out)
    if fmt not in (FMT_NVFP4, FMT_FP8_B128) and log2_scale is not None:
        for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            gen = generator(seed, f"{tag}/{name}", device)
            q = torch.randint(0, 256, (E, N, K // 2), generator=gen, device=device, dtype=torch.int32)
            out[name + "_q"] = q.to(torch.uint8)
            s = _log2_uniform((E, N, K // g), log2_scale[0], log2_scale[1], gen, device)
            if fmt == FMT_ASYM_G64:
                m = -s * (torch.rand((E, N, K // g), generator=gen, device=device) * 3.0 + 6.0)
                out[name + "_sm"] = torch.stack([f16_bits(s), f16_bits(m)], dim=-1).contiguous()
            else:
                out[name + "_sm"] = f16_bits(s).contiguous()
        return Layer(fmt=fmt, num_experts=E, hidden=H, inter=I, **out)
    if fmt == FMT_NVFP4:
        for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            gen = generator(seed, f"{tag}/{name}", device)
            q = torch.randint(0, 256, (E, N, K // 2), generator=gen, device=device, dtype=torch.int32)
            out[name + "_q"] = q.to(torch.uint8)
            # E4M3 scales 0.25 .. 2 (codes 0x28 .. 0x40)
            sb = torch.randint(0x28, 0x41, (E, N, K // 16), generator=gen, device=device, dtype=torch.int32)
            out[name + "_sm"] = sb.to(torch.uint8)
        gen = generator(seed, f"{tag}/global", device)
        glob = torch.rand((E, 2), generator=gen, device=device) * 0.004 + 0.004
        return Layer(fmt=fmt, num_experts=E, hidden=H, inter=I, global_scale=glob, **out)
    if fmt == FMT_FP8_B128:
        for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            gen = generator(seed, f"{tag}/{name}", device)
            q = torch.randint(0, 256, (E, N, K), generator=gen, device=device, dtype=torch.int32)
            q = torch.where((q & 0x7f) == 0x7f, q - 1, q)  # no NaN codes
            out[name + "_q"] = q.to(torch.uint8)
            out[name + "_sm"] = torch.rand((E, N // 128, K // 128), generator=gen, device=device) * 1e-4 + 5e-5
        return Layer(fmt=fmt, num_experts=E, hidden=H, inter=I, **out)
    for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        gen = generator(seed, f"{tag}/{name}", device)
        q = torch.randint(0, 256, (E, N, K // 2), generator=gen, device=device, dtype=torch.int32)
        out[name + "_q"] = q.to(torch.uint8)
        s = (torch.rand((E, N, K // g), generator=gen, device=device) * 0.004 + 0.004)
        if fmt == FMT_ASYM_G64:
            m = -(torch.rand((E, N, K // g), generator=gen, device=device) * 0.03 + 0.03)
            out[name + "_sm"] = torch.stack([f16_bits(s), f16_bits(m)], dim=-1).contiguous()
        else:
            out[name + "_sm"] = f16_bits(s).contiguous()
    return Layer(fmt=fmt, num_experts=E, hidden=H, inter=I, **out)
