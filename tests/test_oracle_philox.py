"""Pins of the oracle's Philox4x32-10 uniforms and Gumbel noise."""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    # the only independent pin of the oracle's Philox: a missing compiler fails the test
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.fail("hipcc is needed to build the rocRAND Philox reference (tests/golden/rocrand_philox_ref.cpp)")
    exe = str(tmp_path_factory.mktemp("rr") / "rocrand_philox_ref")
    src = os.path.join(HERE, "golden", "rocrand_philox_ref.cpp")
    res = subprocess.run([hipcc, "-O1", "--offload-arch=gfx950", "-x", "hip", src, "-o", exe],
                         capture_output=True, text=True)
    if res.returncode != 0:
        pytest.fail("could not build the rocRAND reference: " + res.stderr[-500:])
    return exe


def test_matches_rocrand_engine(rocrand_ref):
    """Oracle Philox4x32-10 == rocRAND's philox4x32_10_engine on random keys and counters."""
    rng = np.random.default_rng(7)
    n = 3000
    seeds = rng.integers(0, 2 ** 63, n, dtype=np.uint64)
    ctr = rng.integers(0, 2 ** 32, (n, 4), dtype=np.uint64)
    ctr[:, 1] >>= 2          # rocRAND reaches word 1 through a 64-bit element offset: < 2^30
    ctr[:10] = 0
    ctr[10:20, 1:] = 0
    seeds[:5] = 0
    lines = "\n".join(f"{int(s)} {c[0]} {c[1]} {c[2]} {c[3]}" for s, c in zip(seeds, ctr)) + "\n"
    out = subprocess.run([rocrand_ref], input=lines, capture_output=True, text=True, check=True).stdout
    ref = np.array([[int(x) for x in ln.split()] for ln in out.strip().splitlines()], dtype=np.uint64)
    for i in range(n):
        s = int(seeds[i])
        got = philox.philox4x32_10(ctr[i].astype(np.uint32)[None], (s & 0xFFFFFFFF, s >> 32))[0]
        assert np.array_equal(got.astype(np.uint64), ref[i]), (i, s, ctr[i])


def test_uniforms_are_exact_odd_multiples():
    u = philox.uniform(1, 0, 0, 0, np.arange(1 << 16))
    assert np.all((u > 0) & (u < 1))
    m = u * 2.0 ** 24
    assert np.all(m == np.floor(m)) and np.all(m % 2 == 1)
    assert np.all(u.astype(np.float32).astype(np.float64) == u)      # exact in fp32
    # extremes of the map
    assert philox.to_uniform(np.array([0], dtype=np.uint32))[0] == 2.0 ** -24
    assert philox.to_uniform(np.array([0xFFFFFFFF], dtype=np.uint32))[0] == 1 - 2.0 ** -24


def test_uniformity_chi_square():
    u = philox.uniform(123, 3, 17, 1, np.arange(1 << 20))
    counts = np.bincount((u * 256).astype(np.int64), minlength=256)
    assert stats.chisquare(counts).pvalue > 1e-4


def test_streams_rows_steps_are_distinct_and_deterministic():
    n = np.arange(4096)
    base = philox.raw_words(9, 0, 5, 0, n)
    assert np.array_equal(base, philox.raw_words(9, 0, 5, 0, n))
    for other in (philox.raw_words(9, 1, 5, 0, n), philox.raw_words(9, 0, 6, 0, n),
                  philox.raw_words(9, 0, 5, 1, n), philox.raw_words(10, 0, 5, 0, n),
                  philox.raw_words(9, 0, 5 + (1 << 32), 0, n)):
        assert np.mean(base == other) < 0.01


def test_counter_layout_groups_four_words():
    """Elements 4m..4m+3 are the four words of one Philox block (counter word 0 = m)."""
    w = philox.raw_words(5, 2, 3, 1, np.arange(8))
    blk = philox.philox4x32_10(np.array([[1, 2, 3, 1]], dtype=np.uint32), (5, 0))[0]
    assert np.array_equal(w[4:8], blk)


def test_gumbel_moments():
    """-ln(-ln U) has mean = Euler-Mascheroni constant and variance pi^2 / 6."""
    g = philox.gumbel(philox.uniform(77, 0, 0, 0, np.arange(1 << 20)))
    assert abs(g.mean() - np.euler_gamma) < 5e-3
    assert abs(g.var() - np.pi ** 2 / 6) < 1e-2
