"""GPU Monte-Carlo marginal (flashhead_mc_marginal) against the oracle, through the C ABI.

FlashHead paper, Appendix D.1 ("Monte-Carlo Simulation"): the sampler's distribution over
the whole vocabulary is estimated by averaging the full conditionals p(v | h, S_i) over N
probe sets drawn like stage 1, and zeros are clipped to the smallest non-zero estimate.
Probe set i uses the stage-1 Philox draws of step i on both sides, so the GPU estimate must
equal oracle.marginal.mc_marginal up to rounding:
  * a probe set is the same on both sides unless the oracle's p-th and (p+1)-th keys are
    within their rounding bounds; such a "flagged" set may differ in its ambiguous
    clusters, and every token those could reach gets an allowance of 1 / N;
  * otherwise each conditional differs only through the logits' rounding: relative error
    at most expm1(2 max|dz| / tau) with |dz| <= gamma(L2) sum_j |h_j e_tj|.
Closed forms pin the GPU path directly too: p = c gives the softmax of z / tau over the
whole vocabulary; the support of the estimate is the union of the forward's probe sets at
steps 0 .. N-1; the unclipped estimate sums to 1.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from clustered_retrieval_lm_amd import flashhead as fh
from clustered_retrieval_lm_amd.head import DeviceHead, to_device
from oracle import head as ohead
from oracle import kmeans, marginal, philox

from . import helpers as H

pytestmark = pytest.mark.gpu


def _oracle_logits(h, h_dtype, C, c_dtype, C2T, tiles, dense_E=None, dense_dtype=None):
    """Centroid logits s, |.| sums, and token logits z (vocabulary order) with their |.| sums."""
    ref1 = ohead.forward(h, h_dtype, C, c_dtype, C2T, tiles, 1, mode="greedy")
    if dense_E is not None:
        dr = ohead.dense_forward(h, h_dtype, dense_E, dense_dtype)
        return ref1.s, ref1.abss, dr.z, dr.absz
    c = C2T.shape[0]
    ref = ohead.forward(h, h_dtype, C, c_dtype, C2T, tiles, c, mode="greedy")
    B = h.shape[0]
    V = C2T.size
    z = np.empty((B, V))
    absz = np.empty((B, V))
    for r in range(B):
        z[r, ref.tokens[r].reshape(-1)] = ref.z[r].reshape(-1)
        absz[r, ref.tokens[r].reshape(-1)] = ref.absz[r].reshape(-1)
    return ref1.s, ref1.abss, z, absz


def _allowance(s, abss, C2T, p, tau, n_sets, seed, row, L1):
    """Per-token allowance for probe sets whose boundary is within rounding, and their count."""
    c, b = C2T.shape
    ks = np.arange(c)
    allow = np.zeros(C2T.size)
    flagged = 0
    if p == c:
        return allow, flagged
    for i in range(n_sets):
        G = philox.gumbel(philox.uniform(seed, row, i, 0, ks))
        key = s / tau + G
        e = H.key_bound(s, abss, L1, True, tau, G)
        order = np.lexsort((ks, -key))
        kp, kq = order[p - 1], order[p]
        if key[kp] - key[kq] <= e[kp] + e[kq]:
            flagged += 1
            lo, hi = key[kq] - e[kq] - e[kp], key[kp] + e[kp] + e[kq]
            amb = (key + e >= lo) & (key - e <= hi)
            reach = amb.copy()
            reach[order[:p]] = True
            allow[C2T[reach].reshape(-1)] += 1.0 / n_sets
    return allow, flagged


def _check_row(got_raw, got_clip, s, abss, z, absz, C2T, p, tau, n_sets, seed, row, L1, L2, max_flag):
    est = marginal.mc_marginal(s, z, C2T, p, tau, n_sets, seed, row=row, clip=False)
    allow, flagged = _allowance(s, abss, C2T, p, tau, n_sets, seed, row, L1)
    assert flagged <= max_flag, f"row {row}: {flagged} probe sets at a rounding tie"
    dz = H.gamma(L2) * np.max(absz)
    rel = np.expm1(2.0 * dz / tau) * 1.01 + 1e-12
    err = np.abs(got_raw - est)
    assert np.all(err <= rel * est + allow + 1e-300), \
        f"row {row}: estimate off by {np.max(err - rel * est - allow):.3g} beyond the bound"
    assert np.all(got_raw >= 0.0)
    assert abs(got_raw.sum() - 1.0) <= 1e-9
    # clipping: zeros become the row's smallest non-zero estimate, nothing else changes (the
    # two calls' fp64 atomic sums may differ in the last bits)
    nz = got_raw > 0
    assert np.all(got_clip > 0)
    assert np.allclose(got_clip[nz], got_raw[nz], rtol=1e-12, atol=0.0)
    assert np.all(got_clip[~nz] == got_clip[nz].min())
    if flagged == 0:
        est_c = marginal.mc_marginal(s, z, C2T, p, tau, n_sets, seed, row=row, clip=True)
        assert np.array_equal(est_c > 0, got_clip > 0)
        assert np.all(np.abs(got_clip - est_c) <= rel * est_c + 1e-300)
    return flagged


def _gpu_mc(dev, h, p, tau, seed, n_sets):
    raw = dev.mc_marginal(h, p, tau=tau, seed=seed, n_sets=n_sets, clip=False)
    clip = dev.mc_marginal(h, p, tau=tau, seed=seed, n_sets=n_sets, clip=True)
    torch.cuda.synchronize()
    return raw.cpu().numpy(), clip.cpu().numpy()


def _tiny(seed, c=8, b=4, d=16):
    rng = np.random.default_rng(seed)
    E = (rng.standard_normal((c * b, d)) * 0.8).astype(np.float32)
    C2T = np.sort(rng.permutation(c * b).reshape(c, b), axis=1).astype(np.int32)
    C = (rng.standard_normal((c, d)) * 0.8).astype(np.float32)
    h = rng.standard_normal((1, d)).astype(np.float32)
    return E, C, C2T, h


@pytest.mark.parametrize("p,tau,seed,n_sets", [(1, 1.0, 1, 2000), (2, 0.7, 2, 1500), (3, 1.3, 3, 1000),
                                               (5, 0.5, 4, 777)])
def test_tiny_head_matches_the_oracle_estimator(gpu, p, tau, seed, n_sets):
    c, b, d = 8, 4, 16
    E, C, C2T, h = _tiny(seed, c, b, d)
    dev = DeviceHead(d, c * b, c, C, C2T, E, "f32", "f32", "f32", "f32", device=gpu)
    raw, clip = _gpu_mc(dev, to_device(h, gpu), p, tau, seed, n_sets)
    tiles = ohead.pack_tiles(E, "f32", C2T, "f32")
    s, abss, z, absz = _oracle_logits(h, "f32", C, "f32", C2T, tiles)
    _check_row(raw[0], clip[0], s[0], abss[0], z[0], absz[0], C2T, p, tau, n_sets, seed, 0,
               H.L_gemv("f32", d), H.L_gemv("f32", d), max_flag=2)


def test_tiny_head_converges_to_the_exact_marginal(gpu):
    """With many probe sets the estimate approaches the enumerated two-stage marginal."""
    c, b, d, p, tau, seed = 8, 4, 16, 3, 0.9, 21
    E, C, C2T, h = _tiny(seed, c, b, d)
    dev = DeviceHead(d, c * b, c, C, C2T, E, "f32", "f32", "f32", "f32", device=gpu)
    n = 200000
    raw, _ = _gpu_mc(dev, to_device(h, gpu), p, tau, seed, n)
    s = C.astype(np.float64) @ h[0].astype(np.float64)
    z = E.astype(np.float64) @ h[0].astype(np.float64)
    P = marginal.two_stage_marginal(s, z, C2T, p, tau)
    # each conditional lies in [0, 1]: the average's standard error is at most 0.5 / sqrt(n)
    assert np.max(np.abs(raw[0] - P)) <= 5 * 0.5 / np.sqrt(n)


def test_all_clusters_give_the_full_softmax(gpu):
    """p = c: every probe set holds the whole vocabulary, so the estimate is softmax(z / tau)."""
    d, b, c, B, tau = 128, 16, 256, 3, 0.8
    hd = workloads.make_small(d, b * c, c, B, seed=5, sigma_c=1.0, sigma_n=0.5, dtype="bf16")
    C2T = H.latent_clusters(hd.latent, c)
    C = kmeans.centroids_from_c2t(ohead.decode(hd.E, "bf16"), C2T, "bf16")
    dev = DeviceHead(d, b * c, c, C, C2T, hd.E, "bf16", "bf16", "bf16", "bf16", device=gpu)
    raw, _ = _gpu_mc(dev, to_device(hd.h, gpu), c, tau, 3, 4)
    dr = ohead.dense_forward(hd.h, "bf16", hd.E, "bf16")
    L2 = max(H.L_gemv("bf16", d), H.L_mfma(d))
    for r in range(B):
        x = dr.z[r] / tau
        P = np.exp(x - x.max())
        P /= P.sum()
        rel = np.expm1(2.0 * H.gamma(L2) * np.max(dr.absz[r]) / tau) * 1.01 + 1e-12
        assert np.all(np.abs(raw[r] - P) <= rel * P + 1e-300)


def test_support_is_the_union_of_the_forward_probe_sets(gpu):
    """The estimate is non-zero exactly on the tokens of the sampler's probe sets at steps
    0 .. N-1 (both are computed on the GPU from the same stage-1 keys)."""
    d, b, c, p, tau, seed, n = 256, 16, 1003, 37, 0.9, 8, 40
    hd = workloads.make_small(d, b * c, c, 1, seed=17, sigma_c=1.0, sigma_n=0.5, dtype="bf16")
    C2T = H.latent_clusters(hd.latent, c)
    C = kmeans.centroids_from_c2t(ohead.decode(hd.E, "bf16"), C2T, "bf16")
    dev = DeviceHead(d, b * c, c, C, C2T, hd.E, "bf16", "bf16", "bf16", "bf16", device=gpu)
    h = to_device(hd.h, gpu)
    for n_sets in (1, n):
        raw, _ = _gpu_mc(dev, h, p, tau, seed, n_sets)
        reached = np.zeros(c, dtype=bool)
        for step in range(n_sets):
            out = dev.forward(h, p, mode="sample", tau=tau, seed=seed, step=step)
            reached[out["probe_ids"].cpu().numpy()[0]] = True
        want = np.zeros(b * c, dtype=bool)
        want[C2T[reached].reshape(-1)] = True
        assert np.array_equal(raw[0] > 0, want)


SMALL = [
    # d, b, c, B, p, dtype, e_dtype, tau, n_sets
    (128, 16, 1024, 1, 32, "bf16", "bf16", 1.0, 300),
    (136, 16, 1003, 3, 37, "bf16", "bf16", 0.7, 200),     # ragged c, B > 1 (Philox row = batch row)
    (96, 16, 300, 2, 20, "f32", "f32", 1.0, 250),
    (512, 16, 400, 2, 33, "bf16", "int4", 0.9, 200),      # int4 tiles
    (64, 4, 3000, 1, 60, "bf16", "bf16", 1.0, 100),       # 2048 < c <= 4096: two key blocks per thread
    (64, 4, 5000, 1, 100, "bf16", "bf16", 1.2, 100),      # c <= 8192: four key blocks per thread
    (64, 2, 20000, 1, 300, "bf16", "bf16", 1.0, 40),      # c > 16384
    # p large enough that the candidates would not fit the LDS list: keys in registers
    (64, 4, 3000, 1, 1400, "bf16", "bf16", 1.0, 30),      # two key blocks per thread
    (64, 4, 5000, 1, 1500, "bf16", "bf16", 1.0, 30),      # four key blocks per thread
    (64, 2, 20000, 1, 1300, "bf16", "bf16", 1.0, 20),     # c > 16384: 1024-thread workgroups
]


@pytest.mark.parametrize("d,b,c,B,p,dt,et,tau,n_sets", SMALL)
def test_small_heads_match_the_oracle_estimator(gpu, d, b, c, B, p, dt, et, tau, n_sets):
    V = b * c
    hd = workloads.make_small(d, V, c, B, seed=300 + d + c + B, sigma_c=1.0, sigma_n=0.5, dtype=dt)
    C2T = H.latent_clusters(hd.latent, c)
    C = kmeans.centroids_from_c2t(ohead.decode(hd.E, dt), C2T, dt)
    dev = DeviceHead(d, V, c, C, C2T, hd.E, dt, dt, et, dt, device=gpu)
    seed = 11
    raw, clip = _gpu_mc(dev, to_device(hd.h, gpu), p, tau, seed, n_sets)
    tiles = ohead.pack_tiles(hd.E, dt, C2T, et)
    s, abss, z, absz = _oracle_logits(hd.h, dt, C, dt, C2T, tiles)
    L1 = H.L_stage1(B, dt, dt, d)
    L2 = max(H.L_gemv(et, d), H.L_mfma(d))     # z: dense GEMV, bf16 MFMA (B > 1) or int4 tiles
    for r in range(B):
        _check_row(raw[r], clip[r], s[r], abss[r], z[r], absz[r], C2T, p, tau, n_sets, seed, r, L1, L2,
                   max_flag=max(2, n_sets // 50))


def test_outlier_centroid_forces_the_full_selection(gpu):
    """One centroid logit far above the rest stretches the key range the threshold grid spans,
    so the chosen threshold lets far more than the LDS list holds through: every probe set
    then runs the full selection on recomputed keys, and must still match the oracle."""
    d, b, c, p, tau, seed, n_sets = 16, 2, 20000, 100, 1.0, 3, 12
    rng = np.random.default_rng(99)
    h = np.zeros((1, d), dtype=np.float32)
    h[0, 0] = 1.0                                   # s_k = C[k][0] exactly
    C = (rng.standard_normal((c, d)) * 0.01).astype(np.float32)
    C[0, 0] = 1590.0                                # outlier: grid spacing ~6.3 key units
    C[1, 0] = -2.5                                  # lowest grid point -5.5, next 0.83
    E = (rng.standard_normal((c * b, d)) * 0.8).astype(np.float32)
    C2T = np.sort(rng.permutation(c * b).reshape(c, b), axis=1).astype(np.int32)
    s64 = C.astype(np.float64) @ h[0].astype(np.float64)
    ks = np.arange(c)
    above = [int(np.sum(s64 / tau + philox.gumbel(philox.uniform(seed, 0, i, 0, ks)) >= 0.83))
             for i in range(n_sets)]
    assert min(above) > 2048                        # the premise: the list would overflow
    dev = DeviceHead(d, c * b, c, C, C2T, E, "f32", "f32", "f32", "f32", device=gpu)
    raw, clip = _gpu_mc(dev, to_device(h, gpu), p, tau, seed, n_sets)
    tiles = ohead.pack_tiles(E, "f32", C2T, "f32")
    s, abss, z, absz = _oracle_logits(h, "f32", C, "f32", C2T, tiles)
    _check_row(raw[0], clip[0], s[0], abss[0], z[0], absz[0], C2T, p, tau, n_sets, seed, 0,
               H.L_gemv("f32", d), H.L_gemv("f32", d), max_flag=1)


def test_gemma_shape_matches_the_oracle_estimator(gpu):
    """The Gemma-3-1B head (V = 262144, c = 16384, p = 512) with 64 probe sets."""
    wl, hd, C2T, C = H.load("gemma")
    dev = DeviceHead(wl.d, wl.V, wl.c, C, C2T, hd.E, wl.dtype, wl.dtype, wl.e_pack, wl.dtype, device=gpu)
    n_sets, tau, seed = 64, 1.0, wl.sample_seed
    raw, clip = _gpu_mc(dev, to_device(hd.h, gpu), wl.p, tau, seed, n_sets)
    tiles = H.oracle_tiles("gemma")
    s, abss, z, absz = _oracle_logits(hd.h, wl.dtype, C, wl.dtype, C2T, tiles, dense_E=hd.E, dense_dtype=wl.dtype)
    _check_row(raw[0], clip[0], s[0], abss[0], z[0], absz[0], C2T, wl.p, tau, n_sets, seed, 0,
               H.L_stage1(1, wl.dtype, wl.dtype, wl.d), H.L_gemv(wl.e_pack, wl.d), max_flag=3)


def test_gemma_shape_ten_thousand_sets(gpu):
    """Appendix D.1's N = 10^4 at the Gemma-3-1B shape: a distribution, clipped as stated."""
    wl, hd, C2T, C = H.load("gemma")
    dev = DeviceHead(wl.d, wl.V, wl.c, C, C2T, hd.E, wl.dtype, wl.dtype, wl.e_pack, wl.dtype, device=gpu)
    h = to_device(hd.h, gpu)
    raw, clip = _gpu_mc(dev, h, wl.p, 1.0, wl.sample_seed, 10000)
    est = raw[0]
    assert np.all(est >= 0) and abs(est.sum() - 1.0) <= 1e-9
    # whole clusters are reached or not
    reached = est[C2T] > 0
    assert np.all(reached.all(axis=1) | ~reached.any(axis=1))
    nz = est > 0
    assert np.all(clip[0][~nz] == clip[0][nz].min())
    assert np.allclose(clip[0][nz], est[nz], rtol=1e-12, atol=0.0)
    # the first 64 sets are a prefix of the 10^4: adding sets only adds reached clusters
    raw64, _ = _gpu_mc(dev, h, wl.p, 1.0, wl.sample_seed, 64)
    assert np.all(nz[raw64[0] > 0])


def test_rejects_bad_arguments(gpu):
    c, b, d = 8, 4, 16
    E, C, C2T, h = _tiny(1, c, b, d)
    dev = DeviceHead(d, c * b, c, C, C2T, E, "f32", "f32", "f32", "f32", device=gpu)
    hh = to_device(h, gpu)
    with pytest.raises(fh.FlashHeadError) as ei:
        dev.mc_marginal(hh, 2, tau=1.0, n_sets=0)
    assert ei.value.status == fh.FH_ERR_ARG
    with pytest.raises(fh.FlashHeadError) as ei:
        dev.mc_marginal(hh, 9, tau=1.0, n_sets=10)
    assert ei.value.status == fh.FH_ERR_ARG
    small = torch.empty(64, dtype=torch.uint8, device=gpu)
    with pytest.raises(fh.FlashHeadError) as ei:
        dev.mc_marginal(hh, 2, tau=1.0, n_sets=10, workspace=small)
    assert ei.value.status == fh.FH_ERR_WORKSPACE
