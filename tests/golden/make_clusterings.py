"""Write the oracle's balanced clusterings of the synthetic heads.

Each workload's clusters are defined as the output of the oracle's balanced
spherical k-means (10 iterations, k-means++ from the data seed) on the seeded
synthetic E.  The large heads take minutes of CPU time, so the cluster-to-token
maps are computed once by this script -- which calls only ``oracle`` and the
seeded generator in ``workloads`` -- and stored as
``tests/golden/clusters_<workload>.npz`` (C2T int32[c][16], the k-means++ seed
indices and the final objective).  Centroids are recomputed from C2T by
``oracle.kmeans.centroids_from_c2t`` when a test or benchmark loads them.

usage: python tests/golden/make_clusterings.py [workload ...]
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from oracle import head, kmeans  # noqa: E402

GOLDEN = os.path.dirname(os.path.abspath(__file__))
# int4_b16 shares int4's E (h is drawn after E), hence its clustering.
DEFAULT = ["tiny", "gemma", "llama", "qwen", "int4"]


def path_for(name: str) -> str:
    return os.path.join(GOLDEN, f"clusters_{name}.npz")


def make(name: str) -> None:
    wl = workloads.WORKLOADS[name]
    t0 = time.time()
    hd = workloads.make_head(wl)
    E = head.decode(hd.E, wl.dtype)
    del hd
    _, C2T, info = kmeans.build_clusters(E, wl.c, wl.kmeans_iters, wl.data_seed,
                                         out_dtype=wl.dtype, return_info=True)
    np.savez_compressed(path_for(name), C2T=C2T, init=info["init"].astype(np.int32),
                        objective=np.float64(info["objective"]))
    print(f"{name}: c={wl.c} V={wl.V} d={wl.d} objective={info['objective']:.6f} "
          f"time={time.time() - t0:.1f}s", flush=True)


if __name__ == "__main__":
    for n in (sys.argv[1:] or DEFAULT):
        make(n)
