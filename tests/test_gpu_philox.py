"""The device Philox4x32-10 words and Gumbel values against the oracle's (through the C ABI).

The sampler's cluster keys (stream 0), token keys (stream 1) and the k-means++ draws (stream 2)
all come from the counter layout that flashhead_philox_words exposes; the words must be equal
bit for bit to oracle.philox.raw_words over more than 10^6 counters, and the fp32 Gumbel values
G = -ln(-ln u) within the bound eps_G = 2^-20 (1 + |G|) that the parity tests' key bounds
assume, checked over 10^7 uniforms.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from clustered_retrieval_lm_amd import flashhead as fh
from oracle import philox

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,row,step,stream,n0,count", [
    (1, 0, 0, 0, 0, 1 << 20),                   # cluster keys of row 0, step 0: 2^20 counters
    (1, 0, 0, 1, 0, 1 << 20),                   # token keys
    (0, 0, 7, 2, 0, 4096),                      # k-means++ draws
    (0xDEADBEEF12345678, 63, 999, 1, 262144 - 4096, 8192),
    (5, 3, (1 << 32) + 17, 0, 0xFFFFFFFF - 1000, 1001),   # high step word, n up to 2^32 - 1
])
def test_words_bit_exact(gpu, seed, row, step, stream, n0, count):
    w = torch.empty(count, dtype=torch.int32, device=gpu)
    fh.flashhead_philox_words(seed, row, step, stream, n0, count, words_out=w)
    torch.cuda.synchronize()
    got = w.cpu().numpy().view(np.uint32)
    want = philox.raw_words(seed, row, step, stream, np.arange(n0, n0 + count, dtype=np.int64))
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} words differ, first at n = {n0 + bad[0]}"


def test_gumbel_within_eps_g(gpu):
    """fp32 -ln(-ln u) on the device within 2^-20 (1 + |G|) of the fp64 value, over 10^7 uniforms."""
    n = 10_000_000
    g = torch.empty(n, dtype=torch.float32, device=gpu)
    w = torch.empty(n, dtype=torch.int32, device=gpu)
    fh.flashhead_philox_words(11, 2, 3, 0, 0, n, words_out=w, gumbel_out=g)
    torch.cuda.synchronize()
    words = w.cpu().numpy().view(np.uint32)
    ref = philox.gumbel(philox.to_uniform(words))
    got = g.cpu().numpy().astype(np.float64)
    ratio = np.abs(got - ref) / (2.0 ** -20 * (1.0 + np.abs(ref)))
    print(f"max |G_gpu - G| / eps_G = {ratio.max():.3g}")
    assert ratio.max() <= 1.0
    # the extremes of the uniform map are reached without overflow
    u = philox.to_uniform(np.array([0, 0xFFFFFFFF], dtype=np.uint32))
    assert np.all(np.isfinite(philox.gumbel(u)))
