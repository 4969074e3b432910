"""Pins of the oracle's balanced spherical k-means (FlashHead paper, Section 3.1)."""
from __future__ import annotations

import os

import numpy as np
import pytest
from scipy import stats

import workloads
from oracle import codecs, kmeans, philox
from oracle import head as ohead

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _check_balanced(C2T: np.ndarray, V: int, c: int) -> None:
    b = V // c
    assert C2T.shape == (c, b)
    assert np.array_equal(np.sort(C2T.reshape(-1)), np.arange(V)), "C2T is not a permutation of [0, V)"
    assert np.all(np.diff(C2T, axis=1) > 0), "tokens of a cluster not in ascending id order"


@pytest.mark.parametrize("V,c,d,seed", [(64, 8, 5, 0), (96, 32, 7, 1), (120, 40, 3, 2), (50, 50, 4, 3), (48, 1, 6, 4)])
def test_every_cluster_has_exactly_v_over_c_tokens(V, c, d, seed):
    rng = np.random.default_rng(seed)
    E = rng.standard_normal((V, d))
    E[3] = 0.0                      # a zero row stays a valid member
    cent, C2T = kmeans.build_clusters(E, c, iters=4, seed=seed)
    _check_balanced(C2T, V, c)
    assert cent.shape == (c, d)


def test_c_must_divide_v():
    with pytest.raises(ValueError):
        kmeans.build_clusters(np.ones((10, 2)), 3)


def test_tiny_head_recovers_latent_partition_and_matches_stored():
    """Well separated latent clusters (256 x 16, sigma_n = 0.3) are recovered exactly."""
    wl = workloads.WORKLOADS["tiny"]
    hd = workloads.make_head(wl)
    E = ohead.decode(hd.E, "f32")
    cent, C2T = kmeans.build_clusters(E, wl.c, wl.kmeans_iters, wl.data_seed, out_dtype="f32")
    _check_balanced(C2T, wl.V, wl.c)
    for k in range(wl.c):
        assert len(set(hd.latent[C2T[k]].tolist())) == 1
    stored = np.load(os.path.join(GOLDEN, "clusters_tiny.npz"))["C2T"]
    assert np.array_equal(stored, C2T)


def test_balanced_assign_reduces_to_argmax_when_nothing_overflows():
    rng = np.random.default_rng(5)
    c, b, d = 6, 4, 6
    Cn = np.eye(d)[:c]
    E = np.repeat(Cn, b, axis=0) + 0.05 * rng.standard_normal((c * b, d))
    En = E / np.linalg.norm(E, axis=1, keepdims=True)
    a = kmeans.balanced_assign(En, Cn, b)
    assert np.array_equal(a, np.repeat(np.arange(c), b))


def test_balanced_assign_evicts_least_similar_member():
    """Cluster 0 is over-full by one: its least similar member moves to the cluster with room."""
    Cn = np.array([[1.0, 0.0], [0.0, 1.0]])
    E = np.array([[1.0, 0.1], [1.0, 0.3], [1.0, 0.2], [0.1, 1.0]])
    En = E / np.linalg.norm(E, axis=1, keepdims=True)
    assert np.array_equal(kmeans.balanced_assign(En, Cn, 2), [0, 1, 0, 1])


def test_balanced_assign_repair_order_and_ties():
    """Evicted tokens go, in ascending id, to their most similar cluster that has room."""
    # three centroids on the unit circle at 0, 120 and 240 degrees
    ang = np.deg2rad([0.0, 120.0, 240.0])
    Cn = np.stack([np.cos(ang), np.sin(ang)], axis=1)
    # five tokens near centroid 0, one near centroid 2; b = 2
    deg = np.array([2.0, -40.0, 1.0, 50.0, -3.0, 235.0])
    E = np.stack([np.cos(np.deg2rad(deg)), np.sin(np.deg2rad(deg))], axis=1)
    a = kmeans.balanced_assign(E, Cn, 2)
    # cluster 0 keeps the two closest (tokens 2 at 1 deg and 0 at 2 deg); evicted in id order:
    # 1 (-40 deg: closer to 240 than 120) -> 2; 3 (50 deg) -> 1; 4 (-3 deg) -> 1 (2 is full)
    assert np.array_equal(a, [0, 2, 0, 1, 1, 2])
    # exact duplicates: the smaller token id is kept
    E2 = np.array([[1.0, 0.0], [1.0, 0.0], [0.0, 1.0], [1.0, 0.0]])
    a2 = kmeans.balanced_assign(E2, np.array([[1.0, 0.0], [0.0, 1.0]]), 2)
    assert np.array_equal(a2, [0, 0, 1, 1])


def test_kmeanspp_picks_every_point_once_when_c_equals_v():
    rng = np.random.default_rng(2)
    En = rng.standard_normal((40, 5))
    En /= np.linalg.norm(En, axis=1, keepdims=True)
    chosen = kmeans.kmeanspp_init(En, 40, seed=3)
    assert np.array_equal(np.sort(chosen), np.arange(40))


def test_kmeanspp_second_pick_follows_d2_weights():
    """With the first centre fixed, the second is drawn with probability w_i / sum w."""
    pts = np.deg2rad(np.array([0.0, 30.0, 90.0, 150.0, 200.0]))
    En = np.stack([np.cos(pts), np.sin(pts)], axis=1)
    counts = np.zeros(5)
    firsts = []
    n = 4000
    for seed in range(n):
        ch = kmeans.kmeanspp_init(En, 2, seed)
        firsts.append(ch[0])
        if ch[0] == 0:
            counts[ch[1]] += 1
    # first centre is floor(u V): uniform over the 5 points
    assert stats.chisquare(np.bincount(firsts, minlength=5)).pvalue > 1e-4
    w = 2.0 - 2.0 * (En @ En[0])
    w[0] = 0.0
    expected = w / w.sum() * counts.sum()
    assert counts[0] == 0
    assert stats.chisquare(counts[1:], expected[1:]).pvalue > 1e-4


def test_centroids_are_member_means_rounded_once():
    E = np.array([[1.0, 2.0], [2.0, 4.0], [4.0, 0.0], [0.0, 1.0], [1.0, 1.0], [1.0, 0.0]])
    C2T = np.array([[0, 1, 2], [3, 4, 5]])
    c32 = kmeans.centroids_from_c2t(E, C2T, "f32")
    assert np.array_equal(c32, np.array([[7 / 3, 2.0], [2 / 3, 2 / 3]], dtype=np.float32))
    cbf = kmeans.centroids_from_c2t(E, C2T, "bf16")
    assert np.array_equal(cbf, codecs.round_to_bf16(np.array([[7 / 3, 2.0], [2 / 3, 2 / 3]])))


def test_objective_zero_for_pure_direction_clusters():
    E = np.array([[2.0, 0.0], [0.5, 0.0], [0.0, 3.0], [0.0, 1.0]])
    En = E / np.linalg.norm(E, axis=1, keepdims=True)
    assert abs(kmeans.objective(En, np.array([0, 0, 1, 1]), 2)) < 1e-12
    assert kmeans.objective(En, np.array([0, 1, 0, 1]), 2) > 0.5


@pytest.mark.parametrize("name", ["gemma", "llama", "qwen", "int4"])
def test_stored_large_clusterings_are_balanced(name):
    """The stored oracle clusterings of the large heads (parity unpinned beyond these invariants)."""
    path = os.path.join(GOLDEN, f"clusters_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    wl = workloads.WORKLOADS[name]
    C2T = np.load(path)["C2T"]
    _check_balanced(C2T, wl.V, wl.c)


def test_kmeanspp_uses_stream_two():
    """The k-means++ draws are Philox stream 2 (row 0, step = draw number)."""
    V = 1000
    En = np.eye(V)[:, :8].copy()
    En[:, 0] = 1.0
    En /= np.linalg.norm(En, axis=1, keepdims=True)
    first = kmeans.kmeanspp_init(En, 1, seed=11)[0]
    assert first == int(np.floor(philox.uniform(11, 0, 0, 2, 0) * V))


def test_unit_centroids_are_normalised_sums_of_unit_rows():
    """unit=True stores c_k = sum of the members' unit rows, normalised (Section 3.1's centroid).

    Rows with integer coordinates and known norms, so every value is written out by hand:
    cluster 0 holds (3, 4, 0) (norm 5) and (0, 0, 2) (norm 2): unit rows (0.6, 0.8, 0) and
    (0, 0, 1), sum (0.6, 0.8, 1), norm sqrt(2).  Cluster 1 holds (0, 5, 12) (norm 13) and
    (8, 0, 6) (norm 10): unit rows (0, 5/13, 12/13) and (0.8, 0, 0.6).  A raw sum, a mean or
    a sum of raw rows normalised once would all differ from these.
    """
    E = np.array([[3.0, 4.0, 0.0], [0.0, 5.0, 12.0], [0.0, 0.0, 2.0], [8.0, 0.0, 6.0]])
    C2T = np.array([[0, 2], [1, 3]])
    s0 = np.array([0.6, 0.8, 1.0])
    s1 = np.array([0.8, 5.0 / 13.0, 12.0 / 13.0 + 0.6])
    want = np.stack([s0 / np.sqrt(2.0), s1 / np.sqrt(s1 @ s1)])
    got = kmeans.centroids_from_c2t(E, C2T, "f32", unit=True)
    assert np.array_equal(got, want.astype(np.float32))
    gotb = kmeans.centroids_from_c2t(E, C2T, "bf16", unit=True)
    assert np.array_equal(gotb, codecs.round_to_bf16(want))
    # the mean would be (1.5, 2, 1) for cluster 0: the flag really changes the result
    assert not np.allclose(kmeans.centroids_from_c2t(E, C2T, "f32"), got)
    # a zero row has no direction: it adds nothing to its cluster's sum
    E0 = np.array([[3.0, 4.0, 0.0], [0.0, 0.0, 0.0]])
    got0 = kmeans.centroids_from_c2t(E0, np.array([[0, 1]]), "f32", unit=True)
    assert np.array_equal(got0, np.array([[0.6, 0.8, 0.0]], dtype=np.float32))


def test_build_clusters_unit_stores_the_unit_centroids_of_its_clustering():
    """build_clusters(unit=True) stores normalise(sum of unit member rows) of the C2T it returns.

    Two tight groups of rows along orthogonal axes (b = 3): the clustering is forced, and the
    stored centroids must equal the hand-computed normalised sums of the unit rows."""
    E = np.array([[2.0, 0.1, 0.0], [0.0, 3.0, 0.2], [4.0, 0.0, 0.3], [0.1, 1.0, 0.0],
                  [1.0, 0.2, 0.1], [0.2, 2.0, 0.1]])
    stored, C2T = kmeans.build_clusters(E, 2, iters=3, seed=0, unit=True, out_dtype="f32")
    assert sorted(C2T.tolist()) == [[0, 2, 4], [1, 3, 5]]
    for k in range(2):
        g = C2T[k]
        u = E[g] / np.linalg.norm(E[g], axis=1, keepdims=True)
        s = u.sum(axis=0)
        want = (s / np.linalg.norm(s)).astype(np.float32)
        assert np.allclose(stored[k], want, rtol=0, atol=2.0 ** -23), (k, stored[k], want)
    # and it agrees with centroids_from_c2t(unit=True) on the returned clustering
    assert np.allclose(stored, kmeans.centroids_from_c2t(E, C2T, "f32", unit=True), rtol=0, atol=2.0 ** -23)
