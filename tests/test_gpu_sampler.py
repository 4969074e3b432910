"""The GPU two-stage sampler against its distribution, through the C ABI.

FlashHead paper, Section 3.2 (stochastic decoding): p clusters drawn without replacement
from softmax(s / tau), then one token from the softmax of z / tau over the gathered tokens.
On tiny heads the exact marginal is enumerated by the oracle (oracle.marginal); the GPU's
token frequencies over many independent draws (distinct Philox rows or steps) must pass a
chi-square test against it.  At the Gemma-3-1B shape, 1000 decode steps are checked for
internal consistency (the token is the Gumbel-max of the probed logits the GPU reports)
and a sample of steps against the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch
from scipy import stats

import workloads
from clustered_retrieval_lm_amd import flashhead as fh
from clustered_retrieval_lm_amd.head import DeviceHead, to_device
from oracle import head as ohead
from oracle import marginal, philox

from . import helpers as H

pytestmark = pytest.mark.gpu


def _chi2_pvalue(counts: np.ndarray, probs: np.ndarray) -> float:
    n = counts.sum()
    exp = probs * n
    order = np.argsort(exp)
    # pool the rarest outcomes until every cell expects >= 5
    cells_o, cells_e, acc_o, acc_e = [], [], 0.0, 0.0
    for i in order:
        acc_o += counts[i]
        acc_e += exp[i]
        if acc_e >= 5.0:
            cells_o.append(acc_o)
            cells_e.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0 and cells_e:
        cells_o[-1] += acc_o
        cells_e[-1] += acc_e
    o, e = np.asarray(cells_o), np.asarray(cells_e)
    chi2 = float(np.sum((o - e) ** 2 / e))
    return float(stats.chi2.sf(chi2, len(o) - 1))


def _tiny_head(seed: int, c=8, b=4, d=16):
    rng = np.random.default_rng(seed)
    V = c * b
    E = (rng.standard_normal((V, d)) * 0.8).astype(np.float32)
    C2T = rng.permutation(V).reshape(c, b)
    C2T.sort(axis=1)
    C = (rng.standard_normal((c, d)) * 0.8).astype(np.float32)
    h = rng.standard_normal((1, d)).astype(np.float32)
    return E, C, C2T.astype(np.int32), h


@pytest.mark.parametrize("p,tau,seed", [(1, 1.0, 1), (2, 0.7, 2), (3, 1.3, 3)])
def test_batched_sampler_matches_the_two_stage_marginal(gpu, p, tau, seed):
    c, b, d = 8, 4, 16
    E, C, C2T, h = _tiny_head(seed, c, b, d)
    dev = DeviceHead(d, c * b, c, C, C2T, E, "f32", "f32", "f32", "f32", device=gpu)
    B = 4096
    hb = to_device(np.repeat(h, B, axis=0), gpu)
    toks = []
    for step in range(5):
        out = dev.forward(hb, p, mode="sample", tau=tau, seed=seed, step=step, probes=False)
        toks.append(out["token"].cpu().numpy())
    toks = np.concatenate(toks)
    s = (C.astype(np.float64) @ h[0].astype(np.float64))
    z = (E.astype(np.float64) @ h[0].astype(np.float64))
    P = marginal.two_stage_marginal(s, z, C2T, p, tau)
    counts = np.bincount(toks, minlength=c * b).astype(np.float64)
    assert counts[P == 0].sum() == 0
    assert _chi2_pvalue(counts, P) > 1e-4


@pytest.mark.parametrize("p,tau,seed", [(2, 1.0, 4)])
def test_single_row_sampler_over_steps_matches_the_marginal(gpu, p, tau, seed):
    c, b, d = 8, 4, 16
    E, C, C2T, h = _tiny_head(seed, c, b, d)
    dev = DeviceHead(d, c * b, c, C, C2T, E, "f32", "f32", "f32", "f32", device=gpu)
    h1 = to_device(h, gpu)
    out = dev.outputs(1, p, probes=False)
    n = 3000
    res = torch.empty(n, dtype=torch.int32, device=gpu)
    for step in range(n):
        dev.forward(h1, p, mode="sample", tau=tau, seed=seed, step=step, out=out, probes=False)
        res[step:step + 1].copy_(out["token"])
    toks = res.cpu().numpy()
    s = C.astype(np.float64) @ h[0].astype(np.float64)
    z = E.astype(np.float64) @ h[0].astype(np.float64)
    P = marginal.two_stage_marginal(s, z, C2T, p, tau)
    counts = np.bincount(toks, minlength=c * b).astype(np.float64)
    assert counts[P == 0].sum() == 0
    assert _chi2_pvalue(counts, P) > 1e-4


def test_gemma_sampling_1000_steps(gpu):
    wl, hd, C2T, C = H.load("gemma")
    dev = DeviceHead(wl.d, wl.V, wl.c, C, C2T, hd.E, wl.dtype, wl.dtype, wl.e_pack, wl.dtype, device=gpu)
    h = to_device(hd.h, gpu)
    p, tau, seed = wl.p, 1.0, wl.sample_seed
    out = dev.outputs(1, p)
    steps = 1000
    tok = np.empty(steps, np.int64)
    check = set(np.random.default_rng(0).choice(steps, 25, replace=False).tolist()) | {0, steps - 1}
    tiles = H.oracle_tiles("gemma")
    rep = H.Report()
    L1 = H.L_stage1(1, wl.dtype, wl.dtype, wl.d)
    L2 = H.L_gemv(wl.e_pack, wl.d)
    ref_cache = {}
    for step in range(steps):
        dev.forward(h, p, mode="sample", tau=tau, seed=seed, step=step, out=out)
        got = {k: v.cpu().numpy()[0] for k, v in out.items()}
        tok[step] = got["token"]
        ids = got["probe_ids"]
        assert np.all(np.diff(ids) > 0) and ids[0] >= 0 and ids[-1] < wl.c
        assert np.array_equal(got["probe_tokens"], C2T[ids])
        # the token is the Gumbel-max of the reported logits (host keys in fp64)
        t = got["probe_tokens"].reshape(-1)
        g = philox.gumbel(philox.uniform(seed, 0, step, 1, t))
        key = got["probe_logits"].reshape(-1).astype(np.float64) / tau + g
        top = np.max(key)
        assert got["token"] in t
        assert key[np.flatnonzero(t == got["token"])[0]] >= top - 1e-4 * max(1.0, abs(top))
        if step in check:
            ref = ohead.forward(hd.h, wl.dtype, C, wl.dtype, C2T, tiles, p, mode="sample", tau=tau, seed=seed,
                                step=step)
            H.compare_row(ref, 0, ids, got["probe_logits"], got["probe_tokens"], got["token"], p, L1, L2, True, tau,
                          seed, step, False, rep)
            ref_cache[step] = int(ref.token[0])
    print(rep)
    rep.check_flag_rate()
    # different steps draw different tokens: the sampler is not stuck on one token
    assert len(np.unique(tok)) > 10
