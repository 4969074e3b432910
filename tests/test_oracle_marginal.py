"""Pins of the two-stage sampler's distribution (FlashHead paper, Section 3.2 and App. D.1)."""
from __future__ import annotations

import itertools

import numpy as np
import pytest
from scipy import stats

from oracle import head as ohead
from oracle import marginal


def _instance(seed, c=5, b=2, d=3):
    rng = np.random.default_rng(seed)
    V = c * b
    C = rng.standard_normal((c, d))
    E = rng.standard_normal((V, d)) * 1.5
    h = rng.standard_normal(d)
    C2T = rng.permutation(V).reshape(c, b)
    C2T.sort(axis=1)
    return C, E, h, C2T


def _softmax(x):
    e = np.exp(x - x.max())
    return e / e.sum()


@pytest.mark.parametrize("seed", range(3))
def test_all_clusters_gives_full_softmax(seed):
    C, E, h, C2T = _instance(seed)
    s, z = C @ h, E @ h
    P = marginal.two_stage_marginal(s, z, C2T, p=C.shape[0], tau=0.7)
    assert np.allclose(P, _softmax(z / 0.7), atol=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_single_probe_is_product_form(seed):
    C, E, h, C2T = _instance(seed)
    s, z = C @ h, E @ h
    tau = 1.3
    P = marginal.two_stage_marginal(s, z, C2T, p=1, tau=tau)
    ps = _softmax(s / tau)
    expect = np.zeros_like(z)
    for k in range(C.shape[0]):
        expect[C2T[k]] = ps[k] * _softmax(z[C2T[k]] / tau)
    assert np.allclose(P, expect, atol=1e-13)


def test_marginal_sums_to_one_and_probe_sets_sum_to_one():
    C, E, h, C2T = _instance(4, c=6)
    s, z = C @ h, E @ h
    for p in range(1, 7):
        P = marginal.two_stage_marginal(s, z, C2T, p, 0.9)
        assert abs(P.sum() - 1) < 1e-12 and np.all(P >= 0)
        pS = marginal.probe_set_probs(s, p, 0.9)
        assert len(pS) == len(list(itertools.combinations(range(6), p)))
        assert abs(sum(pS.values()) - 1) < 1e-12


def test_sampler_matches_closed_form_marginal():
    """Gumbel-top-p clusters + Gumbel-max token (the oracle forward) vs the enumeration."""
    C, E, h, C2T = _instance(6, c=5, b=2, d=3)
    c, b = C2T.shape
    p, tau, B = 2, 0.9, 4000
    Cf, Ef, hf = C.astype(np.float32), E.astype(np.float32), h.astype(np.float32)
    tiles = ohead.pack_tiles(Ef, "f32", C2T, "f32")
    H = np.tile(hf, (B, 1))
    toks, sets = [], []
    for step in range(6):
        res = ohead.forward(H, "f32", Cf, "f32", C2T, tiles, p, mode="sample", tau=tau, seed=3, step=step)
        toks.append(res.token)
        sets.extend(tuple(x) for x in res.probe_ids.tolist())
    toks = np.concatenate(toks)
    s = Cf.astype(np.float64) @ hf.astype(np.float64)
    z = Ef.astype(np.float64) @ hf.astype(np.float64)
    P = marginal.two_stage_marginal(s, z, C2T, p, tau)
    counts = np.bincount(toks, minlength=c * b)
    keep = P * toks.size > 5
    assert stats.chisquare(counts[keep], P[keep] * toks.size * counts[keep].sum() / (P[keep] * toks.size).sum()).pvalue > 1e-4
    # probe sets: successive sampling without replacement
    pS = marginal.probe_set_probs(s, p, tau)
    keys = sorted(pS)
    obs = np.array([sum(1 for x in sets if x == k) for k in keys], dtype=float)
    exp = np.array([pS[k] for k in keys]) * len(sets)
    m = exp > 5
    assert stats.chisquare(obs[m], exp[m] * obs[m].sum() / exp[m].sum()).pvalue > 1e-4


def test_monte_carlo_estimator_appendix_d1():
    C, E, h, C2T = _instance(8, c=6, b=2, d=3)
    s, z = C @ h, E @ h
    p, tau = 2, 1.0
    exact = marginal.two_stage_marginal(s, z, C2T, p, tau)
    raw = marginal.mc_marginal(s, z, C2T, p, tau, n_sets=4000, seed=2, clip=False)
    assert abs(raw.sum() - 1) < 1e-12                     # normalised by construction
    assert np.abs(raw - exact).sum() < 0.05               # converges to the marginal
    few = marginal.mc_marginal(s, z, C2T, 1, tau, n_sets=2, seed=2, clip=False)
    clipped = marginal.mc_marginal(s, z, C2T, 1, tau, n_sets=2, seed=2, clip=True)
    assert np.any(few == 0)
    assert np.all(clipped > 0) and clipped.min() == few[few > 0].min()
