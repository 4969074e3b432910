"""GPU parity on degenerate stage-1 keys, where the probe selection must fall back from its
one-histogram fast path to the general selection: every key equal, a long run of equal
keys across the p-th place, p = c, and a few keys far above all the others (the linear
histogram between the key extremes then puts the p-th key in a bin with thousands of others).

The inputs are built so that every score is computed exactly on both sides (h is zero or a
one-hot vector, so each dot product has at most one non-zero term).  Ties are then exact,
the order (larger key first, smaller id on ties) decides them, and the GPU must reproduce
the oracle bit for bit: kept clusters, probe logits and token (FlashHead paper, Section
3.2: top-p clusters by centroid score, argmax over the gathered tokens).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from clustered_retrieval_lm_amd.head import DeviceHead, to_device
from oracle import codecs, kmeans
from oracle import head as ohead

from . import helpers as H

pytestmark = pytest.mark.gpu


def _storage(a: np.ndarray, dt: str) -> np.ndarray:
    return codecs.round_to_bf16(a) if dt == "bf16" else a.astype(np.float32)


def _check_exact(dev: DeviceHead, h: np.ndarray, C: np.ndarray, C2T: np.ndarray, tiles, dt: str, p: int):
    out = dev.forward(to_device(h, dev.device), p)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    ref = ohead.forward(h, dt, C, dt, C2T, tiles, p)
    assert np.array_equal(got["probe_ids"][0], ref.probe_ids[0])
    assert np.array_equal(got["probe_tokens"][0], ref.tokens[0])
    assert np.array_equal(got["probe_logits"][0].astype(np.float64), ref.z[0])
    assert got["token"][0] == ref.token[0]
    # the token-only call (no probe outputs) takes other paths through the selection: the same token
    tok = dev.forward(to_device(h, dev.device), p, probes=False)["token"]
    torch.cuda.synchronize()
    assert int(tok.cpu()[0]) == ref.token[0]
    return got, ref


@pytest.mark.parametrize("c,p,dt", [(1003, 37, "bf16"), (16384, 512, "bf16"), (300, 20, "f32")])
def test_all_keys_equal(gpu, c, p, dt):
    d, b = 64, 16
    hd = workloads.make_small(d, b * c, c, 1, seed=c + p, dtype=dt)
    C2T = H.latent_clusters(hd.latent, c)
    C = _storage(np.random.default_rng(c).standard_normal((c, d)), dt)
    h = np.zeros((1, d), dtype=np.float32 if dt == "f32" else np.uint16)
    dev = DeviceHead(d, b * c, c, C, C2T, hd.E, dt, dt, dt, dt, device=gpu)
    got, _ = _check_exact(dev, h, C, C2T, ohead.pack_tiles(hd.E, dt, C2T, dt), dt, p)
    assert np.array_equal(got["probe_ids"][0], np.arange(p))          # every score is 0
    assert got["token"][0] == C2T[:p].min()                            # every logit is 0


@pytest.mark.parametrize("c,p,run,dt", [(1003, 250, 100, "bf16"), (8016, 256, 300, "bf16"), (16384, 512, 700, "bf16"),
                                        # runs short enough for the one-histogram path: up to 64 tied keys
                                        # at the boundary, many of them kept
                                        (16384, 512, 30, "f32"), (8016, 256, 20, "f32"), (4008, 256, 50, "f32")])
def test_equal_run_across_the_boundary(gpu, c, p, run, dt):
    d, b = 128, 16
    hd = workloads.make_small(d, b * c, c, 1, seed=7 * c + p, dtype=dt)
    C2T = H.latent_clusters(hd.latent, c)
    Cf = np.zeros((c, d))
    Cf[:, 0] = np.arange(c) // run                  # runs of `run` equal integer scores
    C = _storage(Cf, dt)
    hf = np.zeros((1, d))
    hf[0, 0] = 1.0
    h = _storage(hf, dt)
    dev = DeviceHead(d, b * c, c, C, C2T, hd.E, dt, dt, dt, dt, device=gpu)
    got, _ = _check_exact(dev, h, C, C2T, ohead.pack_tiles(hd.E, dt, C2T, dt), dt, p)
    # the kept set: the top runs whole, then the smallest ids of the run holding the p-th key
    order = np.lexsort((np.arange(c), -(np.arange(c) // run)))
    assert np.array_equal(got["probe_ids"][0], np.sort(order[:p]))


@pytest.mark.parametrize("c,dt", [(300, "bf16"), (1003, "f32")])
def test_p_equals_c(gpu, c, dt):
    d, b = 136, 16
    hd = workloads.make_small(d, b * c, c, 1, seed=c, dtype=dt)
    C2T = H.latent_clusters(hd.latent, c)
    Ev = ohead.decode(hd.E, dt)
    C = kmeans.centroids_from_c2t(Ev, C2T, dt)
    dev = DeviceHead(d, b * c, c, C, C2T, hd.E, dt, dt, dt, dt, device=gpu)
    out = dev.forward(to_device(hd.h, gpu), c)
    torch.cuda.synchronize()
    assert np.array_equal(out["probe_ids"].cpu().numpy()[0], np.arange(c))
    # p = c probes every token: the token is the dense head's
    dense = ohead.dense_forward(hd.h, dt, hd.E, dt)
    rep = H.Report()
    ref = ohead.forward(hd.h, dt, C, dt, C2T, ohead.pack_tiles(hd.E, dt, C2T, dt), c)
    got = {k: v.cpu().numpy() for k, v in out.items()}
    H.compare_row(ref, 0, got["probe_ids"][0], got["probe_logits"][0], got["probe_tokens"][0], got["token"][0], c,
                  H.L_stage1(1, dt, dt, d), H.L_gemv(dt, d), False, 1.0, 0, 0, dt == "f32", rep)
    assert ref.token[0] == dense.token[0]


@pytest.mark.parametrize("c,p,n_high,dt", [(16384, 512, 150, "bf16"), (8016, 256, 60, "bf16"), (1003, 100, 20, "f32")])
def test_few_keys_far_above(gpu, c, p, n_high, dt):
    # n_high < p scores far above the rest: the others share the lowest four bins of the
    # 2048-bin histogram between the extremes; the kept set is the n_high, then the largest of the rest
    d, b = 64, 16
    hd = workloads.make_small(d, b * c, c, 1, seed=c + n_high, dtype=dt)
    C2T = H.latent_clusters(hd.latent, c)
    rng = np.random.default_rng(c + p)
    Cf = np.zeros((c, d))
    Cf[:, 0] = (np.arange(c) % 61) / 8.0
    high = rng.choice(c, n_high, replace=False)
    Cf[high, 0] = 4096.0 + 16.0 * np.arange(n_high)
    C = _storage(Cf, dt)
    hf = np.zeros((1, d))
    hf[0, 0] = 1.0
    h = _storage(hf, dt)
    s = ohead.decode(C, dt)[:, 0]
    low = s[np.setdiff1d(np.arange(c), high)]
    assert (low.max() - low.min()) * 2048 < 4 * (s.max() - s.min())   # within four bins' width
    dev = DeviceHead(d, b * c, c, C, C2T, hd.E, dt, dt, dt, dt, device=gpu)
    got, _ = _check_exact(dev, h, C, C2T, ohead.pack_tiles(hd.E, dt, C2T, dt), dt, p)
    assert set(high.tolist()) <= set(got["probe_ids"][0].tolist())


@pytest.mark.parametrize("n_top,dt", [(64, "f32"), (64, "bf16"), (16, "bf16"), (15, "f32")])
def test_one_group_holds_many_kept_keys(gpu, n_top, dt):
    # Stage 1 lists the 16 largest keys of every group of 64 consecutive clusters (d = 64, so
    # c = 16384 takes 64-cluster groups).  Here n_top clusters of group 1 (ids 64 ..) hold the
    # largest keys: with n_top >= 16 the group's list is cut short inside the top p and the
    # selection must fall back to all c keys; with 15 the lists hold the whole top p.  Scores
    # are small integers (exact in bf16 and fp32): the result must be the oracle's bit for bit.
    c, p, d, b = 16384, 100, 64, 16
    hd = workloads.make_small(d, b * c, c, 1, seed=500 + n_top, dtype=dt)
    C2T = H.latent_clusters(hd.latent, c)
    Cf = np.zeros((c, d))
    Cf[:, 0] = (np.arange(c) * 37) % 97
    Cf[64:64 + n_top, 0] = 200.0 + 2.0 * np.arange(n_top)
    C = _storage(Cf, dt)
    hf = np.zeros((1, d))
    hf[0, 0] = 1.0
    h = _storage(hf, dt)
    dev = DeviceHead(d, b * c, c, C, C2T, hd.E, dt, dt, dt, dt, device=gpu)
    got, _ = _check_exact(dev, h, C, C2T, ohead.pack_tiles(hd.E, dt, C2T, dt), dt, p)
    assert set(range(64, 64 + n_top)) <= set(got["probe_ids"][0].tolist())


@pytest.mark.parametrize("c,p", [(1003, 37), (9496, 256), (16384, 512)])
def test_batched_tied_and_one_hot_rows(gpu, c, p):
    """B > 1 (the batched MFMA stage 1, the per-row selection and the per-cluster stage 2): rows
    whose keys all tie (h = 0) and a one-hot row whose keys are single exact products (bf16
    centroids repeat values, so it has ties as well).  Every score and logit is exact on both
    sides, so the probe lists (ascending ids, ties to the smaller id), probe logits and tokens
    must match the oracle bit for bit in every row."""
    d, b, dt = 64, 16, "bf16"
    hd = workloads.make_small(d, b * c, c, 1, seed=c + p + 1, dtype=dt)
    C2T = H.latent_clusters(hd.latent, c)
    C = _storage(np.random.default_rng(c + 1).standard_normal((c, d)), dt)
    h = np.zeros((3, d), dtype=np.uint16)
    h[1, 5] = 0x3F80                               # bf16 1.0
    dev = DeviceHead(d, b * c, c, C, C2T, hd.E, dt, dt, dt, dt, device=gpu)
    tiles = ohead.pack_tiles(hd.E, dt, C2T, dt)
    out = dev.forward(to_device(h, gpu), p)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    ref = ohead.forward(h, dt, C, dt, C2T, tiles, p)
    for r in range(3):
        assert np.array_equal(got["probe_ids"][r], ref.probe_ids[r]), f"row {r}"
        assert np.array_equal(got["probe_tokens"][r], ref.tokens[r]), f"row {r}"
        assert np.array_equal(got["probe_logits"][r].astype(np.float64), ref.z[r]), f"row {r}"
        assert got["token"][r] == ref.token[r], f"row {r}"
    assert np.array_equal(got["probe_ids"][0], np.arange(p)) and np.array_equal(got["probe_ids"][2], np.arange(p))
    tok = dev.forward(to_device(h, gpu), p, probes=False)["token"]
    torch.cuda.synchronize()
    assert np.array_equal(tok.cpu().numpy(), ref.token)
