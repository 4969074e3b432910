"""GPU parity of the offline entry points: cluster centroids and tile packing (bit-exact)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from clustered_retrieval_lm_amd import flashhead as fh
from clustered_retrieval_lm_amd.head import to_device
from oracle import codecs, kmeans
from oracle import head as ohead

from . import helpers as H

pytestmark = pytest.mark.gpu


def _gpu_centroids(d, V, c, E, C2T, src, dst, unit, dev):
    cent = torch.empty(c * d, dtype=torch.int16 if dst == "bf16" else torch.float32, device=dev)
    desc = fh.make_desc(1, d, V, c, src, dst, src)
    fh.flashhead_centroids(desc, src, to_device(E, dev), to_device(np.asarray(C2T, np.int32), dev), cent, unit=unit)
    torch.cuda.synchronize()
    a = cent.cpu().numpy().reshape(c, d)
    return a.view(np.uint16) if dst == "bf16" else a


@pytest.mark.parametrize("src,dst", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32")])
def test_centroid_means_bit_exact(gpu, src, dst):
    hd = workloads.make_small(200, 16 * 300, 300, 1, seed=2, dtype=src)
    C2T = H.latent_clusters(hd.latent, 300)
    got = _gpu_centroids(200, 4800, 300, hd.E, C2T, src, dst, False, gpu)
    ref = kmeans.centroids_from_c2t(ohead.decode(hd.E, src), C2T, dst)
    assert np.array_equal(got, ref)


def test_unit_centroids_within_one_ulp(gpu):
    hd = workloads.make_small(136, 5 * 211, 211, 1, seed=3, dtype="bf16")
    C2T = H.latent_clusters(hd.latent, 211)
    got = _gpu_centroids(136, 1055, 211, hd.E, C2T, "bf16", "bf16", True, gpu)
    ref = kmeans.centroids_from_c2t(ohead.decode(hd.E, "bf16"), C2T, "bf16", unit=True)
    diff = np.abs(got.astype(np.int32) - ref.astype(np.int32))        # same sign: ulp distance
    assert diff.max() <= 1 and np.mean(diff == 0) > 0.99
    norms = np.linalg.norm(codecs.bf16_to_f64(got), axis=1)
    assert np.all(np.abs(norms - 1) < 1e-2)


@pytest.mark.parametrize("name", ["gemma", "int4"])
def test_full_size_centroids_bit_exact(gpu, name):
    wl, hd, C2T, C = H.load(name)
    got = _gpu_centroids(wl.d, wl.V, wl.c, hd.E, C2T, wl.dtype, wl.dtype, False, gpu)
    assert np.array_equal(got, C)


@pytest.mark.parametrize("src,dst,d", [("bf16", "bf16", 136), ("f32", "f32", 96), ("f32", "bf16", 64),
                                       ("bf16", "int4", 512), ("f32", "int4", 384)])
def test_pack_bit_exact(gpu, src, dst, d):
    c, b = 123, 16
    hd = workloads.make_small(d, c * b, c, 1, seed=d, dtype=src)
    C2T = H.latent_clusters(hd.latent, c)
    ref = ohead.pack_tiles(hd.E, src, C2T, dst)
    desc = fh.make_desc(1, d, c * b, c, src, src, dst)
    rows = c * b
    nbytes = {"f32": 4 * d, "bf16": 2 * d, "int4": d // 2}[dst] * rows
    tiles = torch.empty(nbytes, dtype=torch.uint8, device=gpu)
    scales = torch.empty(rows * (d // 128), dtype=torch.int16, device=gpu) if dst == "int4" else None
    fh.flashhead_pack(desc, src, to_device(hd.E, gpu), to_device(C2T, gpu), tiles, scales)
    torch.cuda.synchronize()
    assert np.array_equal(tiles.cpu().numpy(), np.ascontiguousarray(ref.data).view(np.uint8).reshape(-1))
    if dst == "int4":
        assert np.array_equal(scales.cpu().numpy().view(np.uint16), ref.scales.reshape(-1))


def test_pack_int4_full_size_sampled_clusters(gpu):
    wl, hd, C2T, _ = H.load("int4")
    d, rows = wl.d, wl.V
    desc = fh.make_desc(1, d, wl.V, wl.c, "bf16", "bf16", "int4")
    tiles = torch.empty(rows * d // 2, dtype=torch.uint8, device=gpu)
    scales = torch.empty(rows * (d // 128), dtype=torch.int16, device=gpu)
    fh.flashhead_pack(desc, "bf16", to_device(hd.E, gpu), to_device(C2T, gpu), tiles, scales)
    torch.cuda.synchronize()
    ks = np.random.default_rng(0).choice(wl.c, 300, replace=False)
    q, s = codecs.int4_quantize(ohead.decode(hd.E[C2T[ks].reshape(-1)], "bf16"))
    gt = tiles.view(wl.c, wl.b, d // 2)[torch.as_tensor(ks, device=gpu)].cpu().numpy().reshape(-1, d // 2)
    gs = scales.view(wl.c, wl.b, d // 128)[torch.as_tensor(ks, device=gpu)].cpu().numpy().view(np.uint16)
    assert np.array_equal(gt, q) and np.array_equal(gs.reshape(-1, d // 128), s)


def test_pack_rejects_non_permutation(gpu):
    d, c, b = 64, 10, 4
    E = torch.zeros(c * b * d, dtype=torch.float32, device=gpu)
    C2T = np.arange(c * b, dtype=np.int32)
    C2T[5] = 7                                                   # 7 twice, 5 missing
    tiles = torch.empty(c * b * d * 4, dtype=torch.uint8, device=gpu)
    with pytest.raises(fh.FlashHeadError) as ei:
        fh.flashhead_pack(fh.make_desc(1, d, c * b, c, "f32", "f32", "f32"), "f32", E, to_device(C2T, gpu), tiles)
    assert ei.value.status == fh.FH_ERR_ARG


@pytest.mark.parametrize("unit", [False, True])
def test_int4_centroids_bit_exact(gpu, unit):
    """Stage-1 int4 centroids (selective quantisation, FlashHead paper Section 4.5): the bf16
    centroids quantised per group of 128; the oracle's rounding of the fp64 sums to bf16
    is exact, so the nibbles and scales must match bit for bit (unit: within one bf16 ulp
    before quantisation, so only the mean form is compared exactly)."""
    d, c, b = 384, 211, 16
    hd = workloads.make_small(d, b * c, c, 1, seed=9, dtype="bf16")
    C2T = H.latent_clusters(hd.latent, c)
    desc = fh.make_desc(1, d, b * c, c, "bf16", "int4", "bf16")
    buf = torch.empty(fh.flashhead_centroids_bytes(desc), dtype=torch.uint8, device=gpu)
    fh.flashhead_centroids(desc, "bf16", to_device(hd.E, gpu), to_device(np.asarray(C2T, np.int32), gpu), buf,
                           unit=unit)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    q, sc = kmeans.centroids_from_c2t(ohead.decode(hd.E, "bf16"), C2T, "int4", unit=unit)
    off = (q.size + 255) // 256 * 256                       # the bytes in between are padding
    assert got.size == off + sc.size * 2
    got_q, got_s = got[:q.size].reshape(q.shape), got[off:].view(np.uint16).reshape(sc.shape)
    if not unit:
        assert np.array_equal(got_q, q) and np.array_equal(got_s, sc)
    else:
        assert np.mean(got_q == q) > 0.99 and np.mean(got_s == sc) > 0.99
