"""Logits with ties of signed zeros or of NaN / -inf at the k-th place
(inputs of the routing tie tests; no expected values are made here)."""
from __future__ import annotations

import numpy as np
import torch

NAN_BITS = np.array([0x7fc0, 0xffc0, 0x7f81, 0xffff, 0x7fff, 0xff81], dtype=np.uint16)
NEG_INF, POS_ZERO, NEG_ZERO = 0xff80, 0x0000, 0x8000


def _bf16(vals) -> np.ndarray:
    return torch.from_numpy(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def tie_logits(T: int, E: int, k: int, seed: int) -> np.ndarray:
    """[T][E] bf16 bits with a tie of the kinds above at rank k in every token."""
    rng = np.random.default_rng(seed)
    out = np.empty((T, E), dtype=np.uint16)
    for t in range(T):
        kind = t % 4
        # leaders before the tie; a NaN / -inf tie keeps at least one finite
        # leader, so that the largest selected logit (and every gate) is finite
        lead = int(rng.integers(1, min(3, k if kind < 2 else k - 1) + 1)) if (kind < 2 or k > 1) else 1
        perm = rng.permutation(E)
        leaders, rest = perm[:k - lead], perm[k - lead:]
        row = np.empty(E, dtype=np.uint16)
        row[leaders] = _bf16(1.0 + 0.125 * np.arange(len(leaders)))
        ntie = min(len(rest), lead + 1 + int(rng.integers(0, 4)))  # the tie straddles rank k
        tie, low = rest[:ntie], rest[ntie:]
        if kind in (0, 1):   # -0 / +0; in kind 0 the lowest tied index holds -0, in kind 1 +0
            signs = rng.integers(0, 2, size=ntie).astype(bool)
            first = np.argmin(tie)
            signs[first] = kind == 0
            row[tie] = np.where(signs, NEG_ZERO, POS_ZERO)
            row[low] = _bf16(-1.0 - rng.random(len(low)))
            if kind == 1 and len(low):
                row[low[np.argmin(low)]] = NAN_BITS[t % len(NAN_BITS)]  # a NaN among the losers
        else:                # NaN / -inf; in kind 2 the lowest tied index holds a NaN, in kind 3 -inf
            isnan = rng.integers(0, 2, size=ntie).astype(bool)
            first = np.argmin(tie)
            isnan[first] = kind == 2
            row[tie] = np.where(isnan, NAN_BITS[rng.integers(0, len(NAN_BITS), size=ntie)], NEG_INF)
            row[low] = np.where(rng.integers(0, 2, size=len(low)).astype(bool),
                                NAN_BITS[rng.integers(0, len(NAN_BITS), size=len(low))], NEG_INF)
        out[t] = row
    return out


