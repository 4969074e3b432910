"""Pins of the oracle's dense head, tile packing and FlashHead forward (paper, Section 3)."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
from scipy import stats

import workloads
from oracle import codecs, philox
from oracle import head as ohead

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _int_head(seed=0, c=6, b=3, d=5, B=2):
    """A head with small integer entries: every dot product is exact in fp64 and in Python ints."""
    rng = np.random.default_rng(seed)
    V = c * b
    E = rng.integers(-4, 5, (V, d)).astype(np.float32)
    C = rng.integers(-4, 5, (c, d)).astype(np.float32)
    h = rng.integers(-3, 4, (B, d)).astype(np.float32)
    C2T = rng.permutation(V).reshape(c, b)
    C2T.sort(axis=1)
    return E, C, h, C2T.astype(np.int32)


@pytest.mark.parametrize("seed", range(5))
def test_forward_against_python_integer_brute_force(seed):
    E, C, h, C2T = _int_head(seed)
    c, b = C2T.shape
    p = 3
    tiles = ohead.pack_tiles(E, "f32", C2T, "f32")
    res = ohead.forward(h, "f32", C, "f32", C2T, tiles, p)
    for r in range(h.shape[0]):
        hr = [int(x) for x in h[r]]
        s = [sum(hr[j] * int(C[k][j]) for j in range(len(hr))) for k in range(c)]
        assert [int(x) for x in res.s[r]] == s
        top = sorted(range(c), key=lambda k: (-s[k], k))[:p]
        assert res.probe_ids[r].tolist() == sorted(top)
        best = None
        for k in sorted(top):
            for jj in range(b):
                t = int(C2T[k][jj])
                z = sum(hr[j] * int(E[t][j]) for j in range(len(hr)))
                q = sorted(top).index(k)
                assert res.z[r][q][jj] == z and res.tokens[r][q][jj] == t
                if best is None or (z, -t) > best:
                    best = (z, -t)
        assert res.token[r] == -best[1]


def test_tie_rules_smaller_ids_win():
    # clusters 1 and 3 have identical centroids: at the boundary the smaller id is kept
    d = 4
    C = np.array([[0, 0, 0, 1], [1, 1, 0, 0], [3, 0, 0, 0], [1, 1, 0, 0], [0, 0, 0, 0]], dtype=np.float32)
    h = np.array([[1, 1, 1, 1]], dtype=np.float32)
    b = 2
    E = np.zeros((10, d), dtype=np.float32)
    E[[2, 3, 6, 7]] = 1.0                      # tokens 2, 3, 6, 7 tie at the maximum
    C2T = np.arange(10, dtype=np.int32).reshape(5, b)
    tiles = ohead.pack_tiles(E, "f32", C2T, "f32")
    res = ohead.forward(h, "f32", C, "f32", C2T, tiles, 2)
    assert res.probe_ids[0].tolist() == [1, 2]   # keys: 1, 2, 3, 2, 0 -> cluster 2 (3), then 1 over 3
    assert res.token[0] == 2                       # tokens 2 and 3 of cluster 1 tie: smaller id
    res = ohead.forward(h, "f32", C, "f32", C2T, tiles, 3)
    assert res.probe_ids[0].tolist() == [1, 2, 3] and res.token[0] == 2
    dense = ohead.dense_forward(h, "f32", E, "f32")
    assert dense.token[0] == 2


def test_pack_tiles_gathers_rows_by_c2t():
    rng = np.random.default_rng(3)
    E = rng.standard_normal((12, 8)).astype(np.float32)
    C2T = rng.permutation(12).reshape(4, 3).astype(np.int32)
    t = ohead.pack_tiles(E, "f32", C2T, "f32")
    for k in range(4):
        for j in range(3):
            assert np.array_equal(t.data[k][j], E[C2T[k][j]])
    tb = ohead.pack_tiles(E, "f32", C2T, "bf16")
    assert np.array_equal(tb.data[2][1], codecs.round_to_bf16(E[C2T[2][1]].astype(np.float64)))
    E128 = rng.standard_normal((12, 128)).astype(np.float32)
    t4 = ohead.pack_tiles(E128, "f32", C2T, "int4")
    q, s = codecs.int4_quantize(E128[C2T[1][2]][None].astype(np.float64))
    assert np.array_equal(t4.data[1][2], q[0]) and np.array_equal(t4.scales[1][2], s[0])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_all_probes_equals_dense_head(dtype, mode):
    """p = c keeps every cluster: the token equals the dense head's (same token uniforms)."""
    hd = workloads.make_small(16, 240, 15, 6, seed=4, dtype=dtype)
    C2T = np.random.default_rng(1).permutation(240).reshape(15, 16).astype(np.int32)
    C2T.sort(axis=1)
    C = hd.E[C2T[:, 0]]                           # any centroids will do at p = c
    tiles = ohead.pack_tiles(hd.E, dtype, C2T, dtype)
    for step in range(4):
        res = ohead.forward(hd.h, dtype, C, dtype, C2T, tiles, 15, mode=mode, tau=0.5, seed=9, step=step)
        den = ohead.dense_forward(hd.h, dtype, hd.E, dtype, mode=mode, tau=0.5, seed=9, step=step)
        assert np.array_equal(res.token, den.token)
        # every vocabulary logit appears once
        assert np.array_equal(np.sort(res.tokens.reshape(6, -1), axis=1), np.tile(np.arange(240), (6, 1)))


def test_dense_argmax_against_python_loops():
    E, _, h, _ = _int_head(7, c=10, b=4, d=6, B=3)
    den = ohead.dense_forward(h, "f32", E, "f32")
    for r in range(3):
        z = [sum(int(h[r][j]) * int(E[t][j]) for j in range(6)) for t in range(E.shape[0])]
        assert den.token[r] == max(range(len(z)), key=lambda t: (z[t], -t))


def test_gumbel_max_sampling_follows_softmax():
    """Dense sampling: token frequencies match softmax(z / tau) (chi-square)."""
    rng = np.random.default_rng(0)
    V, d, B = 12, 4, 3000
    E = rng.standard_normal((V, d)).astype(np.float32)
    h1 = rng.standard_normal(d).astype(np.float32)
    h = np.tile(h1, (B, 1))
    tau = 0.8
    den = ohead.dense_forward(h, "f32", E, "f32", mode="sample", tau=tau, seed=21, step=4)
    z = E.astype(np.float64) @ h1.astype(np.float64)
    pz = np.exp((z - z.max()) / tau)
    pz /= pz.sum()
    counts = np.bincount(den.token, minlength=V)
    assert stats.chisquare(counts, pz * B).pvalue > 1e-4


def test_sample_keys_use_token_ids_and_cluster_ids():
    """Sampling keys add Gumbel noise of stream 0 (cluster id) and stream 1 (vocabulary id)."""
    E, C, h, C2T = _int_head(2, c=6, b=3, d=5, B=2)
    tiles = ohead.pack_tiles(E, "f32", C2T, "f32")
    res = ohead.forward(h, "f32", C, "f32", C2T, tiles, 2, mode="sample", tau=2.0, seed=5, step=3)
    for r in range(2):
        g0 = philox.gumbel(philox.uniform(5, r, 3, 0, np.arange(6)))
        assert np.allclose(res.key1[r], res.s[r] / 2.0 + g0, rtol=0, atol=1e-12)
        g1 = philox.gumbel(philox.uniform(5, r, 3, 1, res.tokens[r]))
        assert np.allclose(res.key2[r], res.z[r] / 2.0 + g1, rtol=0, atol=1e-12)


def test_scored_token_count_matches_the_pages_example():
    """README example of the flash-head package: c + p b = 8016 + 256 * 16 = 12,112 of 128,256."""
    fx = json.load(open(os.path.join(GOLDEN, "scored_tokens.json")))
    V, c, p, b = fx["V"], fx["c"], fx["p"], fx["b"]
    assert V == c * b
    d = 8
    rng = np.random.default_rng(0)
    E = rng.standard_normal((V, d)).astype(np.float32)
    C = rng.standard_normal((c, d)).astype(np.float32)
    h = rng.standard_normal((1, d)).astype(np.float32)
    C2T = np.arange(V, dtype=np.int32).reshape(c, b)
    tiles = ohead.pack_tiles(E, "f32", C2T, "f32")
    res = ohead.forward(h, "f32", C, "f32", C2T, tiles, p)
    scored = res.s.shape[1] + res.z[0].size
    assert scored == fx["scored"]
    assert V // scored == fx["reduction_floor"]          # the page states the ratio as 10x


def test_int4_centroids_are_their_dequantised_values():
    """Selective quantisation of stage 1 (FlashHead paper, Section 4.5, Table 5): the int4
    centroids act through their exact values q * s; each group keeps |x - q s| <= s / 2."""
    from oracle import kmeans
    c, b, d = 40, 4, 256
    hd = workloads.make_small(d, b * c, c, 2, seed=21, dtype="bf16")
    C2T = np.arange(b * c).reshape(c, b).astype(np.int32)
    Cq = kmeans.centroids_from_c2t(ohead.decode(hd.E, "bf16"), C2T, "int4")
    Cb = kmeans.centroids_from_c2t(ohead.decode(hd.E, "bf16"), C2T, "bf16")
    deq = ohead.decode(Cq, "int4")
    s = codecs.bf16_to_f64(Cq[1]).repeat(128, axis=1)
    assert np.all(np.abs(codecs.bf16_to_f64(Cb) - deq) <= s / 2 + 1e-300)
    tiles = ohead.pack_tiles(hd.E, "bf16", C2T, "bf16")
    r4 = ohead.forward(hd.h, "bf16", Cq, "int4", C2T, tiles, 7, mode="sample", tau=0.9, seed=3, step=2)
    rf = ohead.forward(hd.h, "bf16", deq.astype(np.float32), "f32", C2T, tiles, 7, mode="sample", tau=0.9, seed=3,
                       step=2)
    assert np.array_equal(r4.s, rf.s) and np.array_equal(r4.probe_ids, rf.probe_ids)
    assert np.array_equal(r4.token, rf.token)
