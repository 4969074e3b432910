"""GPU parity at the edges of the supported shapes, and at the Llama-3.2-1B c/p sweep shapes.

Limits (include/flashhead.h): c up to 32768 clusters (the B = 1 selection then ranks 8192
candidate-list entries, 8 per thread; the batched one holds 8 keys per thread in four-key
blocks), bf16 rows up to d = 4096, fp32
rows up to d = 2048, int4 rows up to d = 8192 (the centroids' format bounds d too, so
d = 8192 needs int4 centroids).  The sweep of the FlashHead paper's Table 7
varies the cluster size at the Llama-3.2-1B head shape (d = 2048, V = 128256): b = 32
(c = 4008) and b = 8 (c = 16032) besides the b = 16 workload.  Each case goes through the
same comparison as the forward tests (fused and staged entry points, every row against the
oracle within the rounding bounds).
"""
from __future__ import annotations

import pytest

import workloads
from clustered_retrieval_lm_amd.head import DeviceHead
from oracle import head as ohead
from oracle import kmeans

from . import helpers as H
from .test_gpu_forward import _run_and_compare

pytestmark = pytest.mark.gpu

LIMITS = [
    # d, b, c, B, p, dtype, e_dtype
    (64, 2, 32768, 1, 600, "bf16", "bf16"),      # the largest c: 8192 list entries at B = 1
    (64, 2, 32768, 3, 300, "bf16", "bf16"),      # ... and 8 four-key blocks per thread at B > 1
    (4096, 16, 300, 1, 20, "bf16", "bf16"),      # the longest bf16 rows: 8 chunk slots per lane
    (4096, 16, 300, 5, 20, "bf16", "bf16"),      # ... through the MFMA stage 1
    (2048, 16, 300, 1, 20, "f32", "f32"),        # the longest fp32 rows: 8 chunk slots per lane
    (2048, 16, 300, 3, 20, "f32", "f32"),
    (4096, 16, 200, 1, 10, "bf16", "int4"),      # int4 rows under bf16 centroids of the longest bf16 d
    (4096, 16, 200, 2, 10, "bf16", "int4"),
]


def _case(gpu, d, b, c, B, p, dt, et, mode, seed):
    hd = workloads.make_small(d, b * c, c, B, seed=seed, sigma_c=1.0, sigma_n=0.5, dtype=dt)
    C2T = H.latent_clusters(hd.latent, c)
    C = kmeans.centroids_from_c2t(ohead.decode(hd.E, dt), C2T, dt)
    dev = DeviceHead(d, b * c, c, C, C2T, hd.E, dt, dt, et, dt, device=gpu)
    tiles = ohead.pack_tiles(hd.E, dt, C2T, et)
    rep = H.Report()
    for step in ([0, 5] if mode == "sample" else [0]):
        _run_and_compare(dev, hd.h, dt, C, C2T, tiles, p, mode, 0.8, 11, step, dt == "f32", rep)
    print(rep)
    rep.check_flag_rate()


@pytest.mark.parametrize("d,b,c,B,p,dt,et", LIMITS)
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_shape_limits(gpu, d, b, c, B, p, dt, et, mode):
    _case(gpu, d, b, c, B, p, dt, et, mode, seed=d + c + B)


@pytest.mark.parametrize("b,c,p,mode", [(32, 4008, 256, "greedy"), (32, 4008, 128, "sample"),
                                        (8, 16032, 512, "greedy"), (8, 16032, 256, "sample")])
def test_sweep_cluster_sizes_at_the_llama_shape(gpu, b, c, p, mode):
    # the sweep's heads: d = 2048, V = 128256, sigma_c = 0.02, sigma_n = 0.01, bf16, B = 1
    d = 2048
    hd = workloads.make_small(d, b * c, c, 1, seed=c + p, sigma_c=0.02, sigma_n=0.01, dtype="bf16")
    C2T = H.latent_clusters(hd.latent, c)
    C = kmeans.centroids_from_c2t(ohead.decode(hd.E, "bf16"), C2T, "bf16")
    dev = DeviceHead(d, b * c, c, C, C2T, hd.E, "bf16", "bf16", "bf16", "bf16", device=gpu)
    tiles = ohead.pack_tiles(hd.E, "bf16", C2T, "bf16")
    rep = H.Report()
    for step in ([0, 3] if mode == "sample" else [0]):
        _run_and_compare(dev, hd.h, "bf16", C, C2T, tiles, p, mode, 1.0, 1, step, False, rep)
    print(rep)
    rep.check_flag_rate()


@pytest.mark.parametrize("B", [1, 2])
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_int4_centroids_and_rows_at_the_longest_d(gpu, B, mode):
    # d = 8192: int4 centroids (stage 1) and int4 token rows (stage 2), 4 chunk slots per lane
    d, b, c, p = 8192, 16, 200, 10
    hd = workloads.make_small(d, b * c, c, B, seed=8192 + B, sigma_c=1.0, sigma_n=0.5, dtype="bf16")
    C2T = H.latent_clusters(hd.latent, c)
    C = kmeans.centroids_from_c2t(ohead.decode(hd.E, "bf16"), C2T, "int4")
    dev = DeviceHead(d, b * c, c, H.centroid_buffer(C, "int4"), C2T, hd.E, "bf16", "int4", "int4", "bf16",
                     device=gpu)
    tiles = ohead.pack_tiles(hd.E, "bf16", C2T, "int4")
    rep = H.Report()
    for step in ([0, 5] if mode == "sample" else [0]):
        _run_and_compare(dev, hd.h, "bf16", C, C2T, tiles, p, mode, 0.8, 11, step, False, rep)
    print(rep)
    rep.check_flag_rate()
