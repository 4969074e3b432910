"""Distribution of the two-stage sampler (oracle side, fp64, tiny inputs).

Two-stage sampling (the FlashHead paper, Section 3.2, "Stochastic / sampling
decoding"): p clusters are drawn without replacement with probabilities
proportional to w_k = exp(s_k / tau), then one token of the gathered clusters
is drawn from the softmax of z / tau over those tokens.  Its marginal is
    P(t) = sum_S P(S) [cluster(t) in S] exp(z_t/tau) / sum_{u in tokens(S)} exp(z_u/tau)
where P(S) sums, over the orderings of S, the successive-draw probabilities
    prod_i w_{k_i} / (W - sum_{j<i} w_{k_j}).
The paper notes that this distribution has no closed form over the whole
vocabulary (Section 5, limitations) -- on tiny inputs it is enumerated here.

Appendix D.1 ("Monte-Carlo Simulation") estimates it by averaging the full
conditional distributions p(v | h, S_i) over N sampled probe sets; tokens that
no S_i reaches get probability 0, which the paper clips to the smallest nonzero
probability of the same context.
"""
from __future__ import annotations

import itertools

import numpy as np

from . import philox


def _softmax(x: np.ndarray) -> np.ndarray:
    m = np.max(x)
    e = np.exp(x - m)
    return e / e.sum()


def probe_set_probs(s: np.ndarray, p: int, tau: float) -> dict:
    """P(S) for every p-subset S of clusters, by enumerating orderings."""
    w = np.exp((s - np.max(s)) / tau)
    W = w.sum()
    out = {}
    for seq in itertools.permutations(range(len(s)), p):
        pr = 1.0
        taken = 0.0
        for k in seq:
            pr *= w[k] / (W - taken)
            taken += w[k]
        key = tuple(sorted(seq))
        out[key] = out.get(key, 0.0) + pr
    return out


def conditional(z: np.ndarray, C2T: np.ndarray, S, tau: float) -> np.ndarray:
    """p(v | h, S) over the whole vocabulary (zero outside the gathered tokens)."""
    V = z.shape[0]
    toks = np.asarray(C2T, dtype=np.int64)[list(S)].reshape(-1)
    out = np.zeros(V)
    out[toks] = _softmax(z[toks] / tau)
    return out


def two_stage_marginal(s: np.ndarray, z: np.ndarray, C2T: np.ndarray, p: int, tau: float) -> np.ndarray:
    """Exact marginal P(t) of the two-stage sampler for one hidden state.

    s: [c] centroid logits, z: [V] token logits (indexed by vocabulary id).
    """
    out = np.zeros(z.shape[0])
    for S, pS in probe_set_probs(s, p, tau).items():
        out += pS * conditional(z, C2T, S, tau)
    return out


def mc_marginal(s: np.ndarray, z: np.ndarray, C2T: np.ndarray, p: int, tau: float, n_sets: int,
                seed: int, row: int = 0, clip: bool = True) -> np.ndarray:
    """Appendix D.1 estimator with N = n_sets Gumbel-top-p probe sets.

    Probe set i uses the stage-1 uniforms of (seed, row, step = i, stream 0).
    """
    c = s.shape[0]
    ks = np.arange(c)
    acc = np.zeros(z.shape[0])
    for i in range(n_sets):
        key = s / tau + philox.gumbel(philox.uniform(seed, row, i, 0, ks))
        S = np.lexsort((ks, -key))[:p]
        acc += conditional(z, C2T, S, tau)
    est = acc / n_sets
    if clip:
        nz = est[est > 0]
        if nz.size:
            est = np.where(est > 0, est, nz.min())
    return est
