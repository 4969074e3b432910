"""Philox4x32-10 uniforms and Gumbel noise (oracle side, NumPy).

Generator: Philox4x32 with 10 rounds, from Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).  One round maps the
counter (x0, x1, x2, x3) under key (k0, k1) to
    (hi(M1*x2) ^ x1 ^ k0,  lo(M1*x2),  hi(M0*x0) ^ x3 ^ k1,  lo(M0*x0))
and the key is advanced by the Weyl constants (W0, W1) between rounds.

Counter layout used by the head (the FlashHead paper, Section 3.2, asks for
random draws at two places -- clusters "sampled without replacement" and a
token "sampled based on the softmax" -- but fixes no generator; this layout is
our reading):
    key     = (seed mod 2^32, seed >> 32)
    counter = (n >> 2, row, step mod 2^32, ((step >> 32) << 2) | stream)
    word    = n & 3
stream 0: cluster keys (n = cluster id), 1: token keys (n = vocabulary id),
2: k-means++ draws (row 0, step = draw number, n = 0).

uniform(x) = (2 * (x >> 9) + 1) * 2^-24 lies in (0, 1) and is exact in fp32.
gumbel(u)  = -ln(-ln u), evaluated here in fp64.
"""
from __future__ import annotations

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = np.uint32(0x9E3779B9)
W1 = np.uint32(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr: np.ndarray, key: tuple) -> np.ndarray:
    """Apply Philox4x32-10 to counters ctr[..., 4] (uint32) under key (k0, k1)."""
    x = np.asarray(ctr, dtype=np.uint32)
    x0 = x[..., 0].astype(np.uint64)
    x1 = x[..., 1].astype(np.uint64)
    x2 = x[..., 2].astype(np.uint64)
    x3 = x[..., 3].astype(np.uint64)
    k0 = np.uint64(key[0] & 0xFFFFFFFF)
    k1 = np.uint64(key[1] & 0xFFFFFFFF)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + np.uint64(W0)) & _MASK32
            k1 = (k1 + np.uint64(W1)) & _MASK32
        p0 = M0 * x0          # < 2^64, exact in uint64
        p1 = M1 * x2
        y0 = (p1 >> np.uint64(32)) ^ x1 ^ k0
        y1 = p1 & _MASK32
        y2 = (p0 >> np.uint64(32)) ^ x3 ^ k1
        y3 = p0 & _MASK32
        x0, x1, x2, x3 = y0, y1, y2, y3
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def raw_words(seed: int, row, step: int, stream: int, n) -> np.ndarray:
    """The 32-bit Philox word for element n of (seed, row, step, stream)."""
    n = np.asarray(n, dtype=np.int64)
    row = np.broadcast_to(np.asarray(row, dtype=np.int64), n.shape)
    ctr = np.empty(n.shape + (4,), dtype=np.uint32)
    ctr[..., 0] = (n >> 2).astype(np.uint32)
    ctr[..., 1] = row.astype(np.uint32)
    ctr[..., 2] = np.uint32(step & 0xFFFFFFFF)
    ctr[..., 3] = np.uint32((((step >> 32) << 2) | stream) & 0xFFFFFFFF)
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    out = philox4x32_10(ctr, key)
    return np.take_along_axis(out, (n & 3)[..., None], axis=-1)[..., 0]


def to_uniform(x: np.ndarray) -> np.ndarray:
    """Map 32-bit words to (0, 1): odd multiples of 2^-24 (exact in fp32 and fp64)."""
    m = (np.asarray(x, dtype=np.uint32) >> np.uint32(9)).astype(np.float64)
    return (2.0 * m + 1.0) * 2.0 ** -24


def uniform(seed: int, row, step: int, stream: int, n) -> np.ndarray:
    return to_uniform(raw_words(seed, row, step, stream, n))


def gumbel(u: np.ndarray) -> np.ndarray:
    """Standard Gumbel noise -ln(-ln u) in fp64."""
    return -np.log(-np.log(np.asarray(u, dtype=np.float64)))
