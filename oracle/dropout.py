"""Counter-based dropout masks for the oracle (test infrastructure only).

[TP-block] sec. 5: inside a tensor-parallel region (attention scores of the
local heads) the activations are split, so every rank needs its own mask
stream (seed + 2718 + tp_rank); outside it (the hidden state after the
attention and after the MLP, replicated on every rank) all ranks must draw
the same mask (the data-parallel seed). A counter-based generator makes the
mask a pure function of (seed, site, element index, offset), so a
recomputation reproduces it.

The generator is Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC 2011), written here from that
definition: a 4 x 32-bit counter and a 2 x 32-bit key; each of the ten rounds
multiplies counter words 0 and 2 by two fixed constants, swaps the halves of
the products into the other words xor-ed with the key, and the key advances by
two Weyl constants between rounds.

Mask of one site over a flat element index i:
    words = Philox(counter = (i >> 2 low 32 bits, i >> 2 high 32 bits, site, offset),
                   key = (seed low 32 bits, seed high 32 bits))
    r = words[i & 3];  keep = r >= floor(p * 2^32)   (an integer decision)
and a kept element is scaled by 1 / (1 - p).
"""
from __future__ import annotations

import numpy as np

MASK32 = np.uint64(0xFFFFFFFF)
_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)

SITE_ATTN = 0          # attention probabilities (inside the TP region)
SITE_HIDDEN_ATTN = 1   # hidden state after the attention block (outside)
SITE_HIDDEN_MLP = 2    # hidden state after the MLP (outside)
TP_SEED_OFFSET = 2718  # [TP-block] sec. 5: tensor-parallel seed = seed + 2718 + tp_rank


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10; all arguments uint32 values (numpy arrays
    or scalars). Returns the four output words as uint64 arrays < 2^32."""
    c0, c1, c2, c3 = (np.asarray(v, np.uint64) & MASK32 for v in (c0, c1, c2, c3))
    k0 = np.uint64(k0) & MASK32
    k1 = np.uint64(k1) & MASK32
    s32 = np.uint64(32)
    for _ in range(10):
        p0 = _M0 * c0          # 32 x 32 -> 64-bit products
        p1 = _M1 * c2
        # new words: (hi(p1) ^ c1 ^ k0, lo(p1), hi(p0) ^ c3 ^ k1, lo(p0)); every
        # operand is below 2^32, so the xors need no mask
        c0, c1, c2, c3 = (p1 >> s32) ^ c1 ^ k0, p1 & MASK32, (p0 >> s32) ^ c3 ^ k1, p0 & MASK32
        k0 = (k0 + _W0) & MASK32
        k1 = (k1 + _W1) & MASK32
    return c0, c1, c2, c3


def threshold(p):
    """Integer drop threshold: an element is dropped when its 32-bit word is
    below floor(p * 2^32) (p in [0, 1))."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return min(int(np.floor(p * 4294967296.0)), 0xFFFFFFFF)


def words(idx, site, seed, offset):
    """The 32-bit word of every flat element index in `idx`."""
    idx = np.asarray(idx, np.uint64)
    g = idx >> np.uint64(2)
    w = philox4x32_10(g & MASK32, g >> np.uint64(32), np.uint64(site), np.uint64(offset),
                      np.uint64(seed) & MASK32, np.uint64(seed) >> np.uint64(32))
    sel = (idx & np.uint64(3)).astype(np.int64)
    return np.choose(sel, w)


def keep_mask(shape, site, seed, offset, p):
    """Boolean keep mask of an array of `shape` whose elements are numbered
    in row-major order."""
    n = int(np.prod(shape))
    return (words(np.arange(n, dtype=np.uint64), site, seed, offset) >=
            np.uint64(threshold(p))).reshape(shape)


def multiplier(shape, site, seed, offset, p):
    """keep / (1 - p) as float64 (all ones when p == 0)."""
    if p == 0.0:
        return np.ones(shape)
    return keep_mask(shape, site, seed, offset, p) / (1.0 - p)


def attn_seed(seed, tp_rank):
    return seed + TP_SEED_OFFSET + tp_rank


def multiplier_range(start, count, site, seed, offset, p):
    """keep / (1 - p) of the flat elements start .. start + count - 1."""
    if p == 0.0:
        return np.ones(count)
    idx = np.arange(start, start + count, dtype=np.uint64)
    return (words(idx, site, seed, offset) >= np.uint64(threshold(p))) / (1.0 - p)


class AttnMult:
    """Dropout multipliers of the attention probabilities [B, nq, S, S]
    (flat index ((b * nq + h) * S + q) * S + k), made one (batch, head)
    slice at a time: mult[b, h] is the [S, S] slice; np.asarray gives all."""

    def __init__(self, B, nq, S, seed, offset, p):
        self.B, self.nq, self.S = B, nq, S
        self.seed, self.offset, self.p = seed, offset, p
        self.shape = (B, nq, S, S)

    def __getitem__(self, bh):
        b, h = bh
        S = self.S
        return multiplier_range((b * self.nq + h) * S * S, S * S, SITE_ATTN, self.seed,
                                self.offset, self.p).reshape(S, S)

    def __array__(self, dtype=None, copy=None):
        a = np.stack([np.stack([self[b, h] for h in range(self.nq)]) for b in range(self.B)])
        return a if dtype is None else a.astype(dtype)
