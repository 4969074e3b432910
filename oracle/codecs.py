"""Number formats used by the head (oracle side).

bf16: 1 sign, 8 exponent, 7 stored mantissa bits (the top half of an IEEE
float32).  Decoding is exact; encoding rounds to the nearest representable
value, ties to the value with an even last mantissa bit.

int4 group-128 (our reading of the low-bit token embeddings the FlashHead paper
discusses in Section 3.2, "Quantization note", and Table 5; the pages give no
format): per token row and per group of 128 consecutive elements along d,
    s = bf16(amax / 7)            amax = max |x| over the group
    q = clamp(rne(x / s), -7, 7)  (s == 0 gives q = 0)
    x_hat = q * s
q is stored as a two's-complement nibble; element 2j sits in the low nibble of
byte j of the row, element 2j+1 in the high nibble.
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_f64(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round real values (float64) to bf16, nearest-even; returns uint16 bits.

    A finite nonzero x = m * 2^e with 0.5 <= |m| < 1 is rounded to a multiple of
    the bf16 quantum 2^(e-8) (8 significant bits), or of 2^-133 below the
    smallest normal 2^-126.  The scaling by a power of two is exact, and
    np.rint rounds halves to even.  Results of magnitude >= 2^128 become inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)                       # |xf| = m 2^e, 0.5 <= m < 1
    qexp = np.maximum(e - 8, -133)            # quantum exponent
    q = np.ldexp(np.ones_like(xf), qexp)
    r = np.rint(xf / q) * q                   # exact scaling, ties to even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, xf), r)
    out[finite] = r[finite]
    out[~finite] = x[~finite]
    bits = out.astype(np.float32).view(np.uint32)   # exact: r has <= 8 significant bits
    bits = np.where(np.isnan(out), np.uint32(0x7FC00000), bits)
    return (bits >> np.uint32(16)).astype(np.uint16)


def round_to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def int4_quantize(x: np.ndarray):
    """Quantise rows x[..., d] (float64 values, d % 128 == 0).

    Returns (packed uint8[..., d/2], scales uint16 bf16 bits[..., d/128]).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % GROUP == 0
    g = x.reshape(x.shape[:-1] + (d // GROUP, GROUP))
    amax = np.abs(g).max(axis=-1)
    s_bits = round_to_bf16(amax / 7.0)
    s = bf16_to_f64(s_bits)
    safe = np.where(s == 0.0, 1.0, s)
    q = np.rint(g / safe[..., None])
    q = np.where(s[..., None] == 0.0, 0.0, q)
    q = np.clip(q, -7, 7).astype(np.int64).reshape(x.shape)
    nib = (q & 0xF).astype(np.uint8)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << np.uint8(4))).astype(np.uint8)
    return packed, s_bits


def int4_dequantize(packed: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    """Exact values q * s (float64) of packed int4 rows."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = (packed & np.uint8(0xF)).astype(np.int64)
    hi = (packed >> np.uint8(4)).astype(np.int64)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    q = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.float64)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    s = bf16_to_f64(s_bits)
    d = q.shape[-1]
    return (q.reshape(q.shape[:-1] + (d // GROUP, GROUP)) * s[..., None]).reshape(q.shape)
