"""Pins of the oracle's bf16 and int4 codecs."""
from __future__ import annotations

import numpy as np
import torch

from oracle import codecs


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_round_to_bf16_matches_torch_on_random_bits():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    finite = np.isfinite(x)
    got = codecs.round_to_bf16(x[finite].astype(np.float64))
    assert np.array_equal(got, _torch_bf16_bits(x[finite]))


def test_round_to_bf16_ties_and_specials():
    # exact halfway cases: low 16 bits == 0x8000, both parities of the kept bit
    hi = np.arange(0, 0x7F7F, 7, dtype=np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    assert np.array_equal(codecs.round_to_bf16(ties.astype(np.float64)), _torch_bf16_bits(ties))
    assert np.array_equal(codecs.round_to_bf16(-ties.astype(np.float64)), _torch_bf16_bits(-ties))
    sp = np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 3.4e38, 1.5e-39, 2.0 ** -126], dtype=np.float32)
    assert np.array_equal(codecs.round_to_bf16(sp.astype(np.float64)), _torch_bf16_bits(sp))
    assert codecs.round_to_bf16(np.array([np.nan]))[0] & 0x7F80 == 0x7F80


def test_bf16_decode_round_trip_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = codecs.bf16_to_f64(bits)
    ok = np.isfinite(v)
    assert np.array_equal(codecs.round_to_bf16(v[ok]), bits[ok])
    # decoding is the top half of the float32 pattern
    assert np.array_equal(v[ok].astype(np.float32).view(np.uint32) >> 16, bits[ok].astype(np.uint32))


def test_int4_closed_form_group():
    """A group holding exact multiples q * s of a bf16 scale s with max |q| = 7 decodes exactly."""
    s = 0.0078125                                       # 2^-7, exact in bf16
    q = np.tile(np.array([-7, -3, 0, 1, 2, 7, 5, -6], dtype=np.float64), 16)
    packed, sb = codecs.int4_quantize((q * s)[None])
    assert codecs.bf16_to_f64(sb)[0, 0] == s
    assert np.array_equal(codecs.int4_dequantize(packed, sb)[0], q * s)
    # nibble order: element 2i low nibble, element 2i+1 high nibble, two's complement
    assert packed[0, 0] == ((-7) & 0xF) | (((-3) & 0xF) << 4)
    assert packed[0, 1] == 0 | (1 << 4)


def test_int4_zero_group_and_round_trip_bound():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 384)) * rng.uniform(0.001, 3, (50, 1))
    x = codecs.bf16_to_f64(codecs.round_to_bf16(x))   # bf16 inputs, as the head stores them
    x[3, 128:256] = 0.0
    packed, sb = codecs.int4_quantize(x)
    s = codecs.bf16_to_f64(sb)
    assert s[3, 1] == 0 and np.all(codecs.int4_dequantize(packed, sb)[3, 128:256] == 0)
    xh = codecs.int4_dequantize(packed, sb)
    err = np.abs(x - xh).reshape(50, 3, 128)
    assert np.all(err <= s[..., None] / 2 + 1e-15)
    # the element of largest magnitude maps to +-7
    q = np.rint(xh.reshape(50, 3, 128) / np.where(s == 0, 1, s)[..., None])
    amax_q = np.take_along_axis(np.abs(q), np.abs(x.reshape(50, 3, 128)).argmax(-1)[..., None], -1)
    assert np.all(amax_q[s > 0] == 7)
    # s is the bf16 rounding of amax / 7
    amax = np.abs(x.reshape(50, 3, 128)).max(-1)
    assert np.array_equal(sb, _torch_bf16_bits((amax / 7.0).astype(np.float32)))
