"""Pins of the oracle's unequal (padded) clusters: the ablation of the FlashHead paper's
Section 3.1 (a C2T padded to the largest cluster when clusters are not equalised) and
Section 4.5 (Table 6, equal versus unequal clusters).  Empty slots (C2T entry -1) gather
nothing: their logit is -inf, their token -1, and they are never chosen."""
from __future__ import annotations

import itertools

import numpy as np
import pytest

import workloads
from oracle import head as ohead
from oracle import kmeans, philox


def _tiny():
    # five clusters of sizes 3, 1, 2, 4, 2 over V = 12 tokens; small integers, every sum exact
    rng = np.random.default_rng(3)
    E = rng.integers(-4, 5, size=(12, 4)).astype(np.float32)
    h = rng.integers(-3, 4, size=(1, 4)).astype(np.float32)
    C = rng.integers(-3, 4, size=(5, 4)).astype(np.float32)
    C2T = np.array([[0, 5, 9, -1], [3, -1, -1, -1], [1, 11, -1, -1], [2, 4, 7, 10], [6, 8, -1, -1]], dtype=np.int32)
    return E, h, C, C2T


def _brute(E, h, C, C2T, p, mode, tau=1.0, seed=0, step=0):
    """The two stages written out with Python loops: cluster keys, the p largest (ties to the
    smaller id), every member's logit, the token of the largest key (ties to the smaller id)."""
    hv = [float(x) for x in h[0]]
    keys = []
    for k in range(C.shape[0]):
        s = sum(hv[j] * float(C[k][j]) for j in range(len(hv)))
        if mode == "sample":
            s = s / tau + float(philox.gumbel(philox.uniform(seed, 0, step, 0, k)))
        keys.append((s, k))
    kept = sorted(k for _, k in sorted(keys, key=lambda t: (-t[0], t[1]))[:p])
    best = None
    for k in kept:
        for t in C2T[k]:
            if t < 0:
                continue
            z = sum(hv[j] * float(E[t][j]) for j in range(len(hv)))
            key = z if mode == "greedy" else z / tau + float(philox.gumbel(philox.uniform(seed, 0, step, 1, int(t))))
            if best is None or key > best[0] or (key == best[0] and t < best[1]):
                best = (key, int(t))
    return kept, best[1]


@pytest.mark.parametrize("p,mode", list(itertools.product([1, 2, 3, 5], ["greedy", "sample"])))
def test_padded_forward_matches_brute_force(p, mode):
    E, h, C, C2T = _tiny()
    tiles = ohead.pack_tiles(E, "f32", C2T, "f32")
    ref = ohead.forward(h, "f32", C, "f32", C2T, tiles, p, mode=mode, tau=0.7, seed=4, step=2)
    kept, tok = _brute(E, h, C, C2T, p, mode, tau=0.7, seed=4, step=2)
    assert list(ref.probe_ids[0]) == kept
    assert int(ref.token[0]) == tok
    # empty slots: -1 token, -inf logit, and exact logits for the members
    for q, k in enumerate(ref.probe_ids[0]):
        for j in range(C2T.shape[1]):
            t = C2T[k][j]
            if t < 0:
                assert ref.tokens[0][q][j] == -1 and ref.z[0][q][j] == -np.inf
            else:
                assert ref.z[0][q][j] == float(np.dot(h[0].astype(np.float64), E[t].astype(np.float64)))


def test_padded_forward_with_every_cluster_is_the_dense_head():
    E, h, C, C2T = _tiny()
    tiles = ohead.pack_tiles(E, "f32", C2T, "f32")
    for mode in ("greedy", "sample"):
        ref = ohead.forward(h, "f32", C, "f32", C2T, tiles, 5, mode=mode, tau=0.9, seed=1, step=7)
        dense = ohead.dense_forward(h, "f32", E, "f32", mode=mode, tau=0.9, seed=1, step=7)
        assert int(ref.token[0]) == int(dense.token[0])


def test_padding_changes_nothing_for_full_clusters():
    """A C2T without empty slots gives the same results as before the padding rules."""
    E, h, C, _ = _tiny()
    C2T = np.arange(12, dtype=np.int32).reshape(4, 3)
    tiles = ohead.pack_tiles(E, "f32", C2T, "f32")
    ref = ohead.forward(h, "f32", C[:4], "f32", C2T, tiles, 2)
    assert np.all(np.isfinite(ref.z)) and np.all(ref.tokens >= 0)


def test_centroids_of_padded_clusters_are_member_means():
    E = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 0.0], [0.0, 6.0]])
    C2T = np.array([[0, 1, 2], [3, -1, -1]])
    got = kmeans.centroids_from_c2t(E, C2T, "f32")
    assert np.array_equal(got, np.array([[3.0, 2.0], [0.0, 6.0]], dtype=np.float32))
    tiles = ohead.pack_tiles(E.astype(np.float32), "f32", C2T, "f32")
    assert np.all(tiles.data[1][1:] == 0.0)


def test_unequal_clusters_generator():
    latent = np.repeat(np.arange(500), 16)[np.random.default_rng(0).permutation(8000)]
    C2T, sizes = workloads.make_unequal_clusters(latent, 500, seed=5)
    assert sizes.sum() == 8000 and sizes.min() >= 1 and sizes.std() > 3
    members = C2T[C2T >= 0]
    assert np.array_equal(np.sort(members), np.arange(8000))
    for k in range(500):
        row = C2T[k]
        assert np.all(row[:sizes[k]] >= 0) and np.all(row[sizes[k]:] == -1)
        assert np.all(np.diff(row[:sizes[k]]) > 0)
