"""Seeded synthetic inputs for the FlashHead output head.

This module is shared by the CPU oracle, the tests and the benchmark.  It holds
only random-number generation and storage-format conversion (fp64 draws rounded
to fp32, or to bf16 through torch's CPU conversion).  None of the method's
arithmetic (clustering, scoring, selection, quantisation, sampling) lives here.

Workload shapes follow the model heads the FlashHead paper evaluates
("FlashHead: Efficient Drop-In Replacement for the Classification Head in
Language Model Inference", Section 4 and Tables 3-7): Llama-3.2-1B
(d=2048, V=128256, c=8016), Gemma-3-1B (d=1152, V=262144), Qwen-3-0.6B
(d=1024, V=151936) and a tiny head for exhaustive checks.  Every head has
clusters of exactly b=16 tokens, so V = 16 c (the paper's Section 3.1 requires
c to divide v).

Recipe (one numpy PCG64 generator per workload, ``default_rng(seed)``; draws
are taken in this fixed order):
  1. latent centres  M[c][d]  ~ N(0, sigma_c^2)
  2. per-token noise N[V][d]  ~ N(0, sigma_n^2)
  3. a row permutation perm of range(V)
  4. hidden states   h[B][d]  ~ N(0, 1)
E_raw[i] = M[i // 16] + N[i];  E = E_raw[perm]  (token i has latent label
perm[i] // 16).  E, C and h are then stored in the workload's dtype.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

CLUSTER_SIZE = 16


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    d: int
    V: int
    c: int
    B: int
    p: int
    sigma_c: float
    sigma_n: float
    dtype: str            # storage dtype of h, C and E before any packing: "f32" | "bf16"
    e_pack: str           # packed token-embedding dtype: "f32" | "bf16" | "int4"
    temperatures: tuple   # sampling temperatures exercised (greedy is always run)
    sample_seed: int = 1  # Philox key for the sampler
    data_seed: int = 0    # PCG64 seed of the generator and k-means++ key
    kmeans_iters: int = 10
    c_pack: str = ""      # stored centroid dtype when it differs from dtype ("int4")

    @property
    def b(self) -> int:
        return self.V // self.c

    @property
    def c_dtype(self) -> str:
        return self.c_pack or self.dtype


# The five head shapes.  B for "int4" is 1 in the headline configuration; the
# batched variant (B=16) is "int4_b16"; "gemma_c4" is the Gemma shape with int4 centroids.
WORKLOADS = {
    "tiny": Workload("tiny", d=64, V=4096, c=256, B=4, p=8, sigma_c=1.0, sigma_n=0.3,
                     dtype="f32", e_pack="f32", temperatures=(1.0,)),
    "llama": Workload("llama", d=2048, V=128256, c=8016, B=1, p=256, sigma_c=0.02, sigma_n=0.01,
                      dtype="bf16", e_pack="bf16", temperatures=()),
    "gemma": Workload("gemma", d=1152, V=262144, c=16384, B=1, p=512, sigma_c=0.02, sigma_n=0.01,
                      dtype="bf16", e_pack="bf16", temperatures=(1.0,)),
    "qwen": Workload("qwen", d=1024, V=151936, c=9496, B=64, p=256, sigma_c=0.02, sigma_n=0.01,
                     dtype="bf16", e_pack="bf16", temperatures=(0.8,)),
    "int4": Workload("int4", d=3072, V=128256, c=8016, B=1, p=256, sigma_c=0.02, sigma_n=0.01,
                     dtype="bf16", e_pack="int4", temperatures=(1.0,)),
    "int4_b16": Workload("int4_b16", d=3072, V=128256, c=8016, B=16, p=256, sigma_c=0.02,
                         sigma_n=0.01, dtype="bf16", e_pack="int4", temperatures=(1.0,)),
    # the Gemma head with int4 stage-1 centroids and bf16 tiles (selective quantisation)
    "gemma_c4": Workload("gemma_c4", d=1152, V=262144, c=16384, B=1, p=512, sigma_c=0.02, sigma_n=0.01,
                         dtype="bf16", e_pack="bf16", temperatures=(1.0,), c_pack="int4"),
}


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float draws to the storage dtype.

    f32 -> float32 array; bf16 -> uint16 array of bf16 bit patterns, rounded by
    torch's CPU float32->bfloat16 conversion (round to nearest even).
    """
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(x32).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def storage_to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float32 (bf16 bits -> float32)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


@dataclasses.dataclass
class HeadData:
    wl: Workload
    E: np.ndarray        # [V][d] token-major, storage dtype (float32 or uint16 bf16 bits)
    h: np.ndarray        # [B][d] storage dtype
    latent: np.ndarray   # [V] int64 latent cluster label of each token


def make_head(wl: Workload, B: Optional[int] = None, seed: Optional[int] = None) -> HeadData:
    """Generate E and h for a workload (recipe in the module docstring)."""
    seed = wl.data_seed if seed is None else seed
    B = wl.B if B is None else B
    rng = np.random.default_rng(seed)
    M = rng.standard_normal((wl.c, wl.d)) * wl.sigma_c
    noise = rng.standard_normal((wl.V, wl.d)) * wl.sigma_n
    perm = rng.permutation(wl.V)
    h = rng.standard_normal((B, wl.d))
    lat = np.arange(wl.V) // CLUSTER_SIZE
    noise += M[lat]
    del M
    E = to_storage(noise[perm], wl.dtype)
    del noise
    return HeadData(wl=wl, E=E, h=to_storage(h, wl.dtype), latent=lat[perm])


def make_hidden(wl: Workload, B: int, seed: int) -> np.ndarray:
    """Extra hidden states h[B][d] ~ N(0,1) from their own PCG64 stream."""
    rng = np.random.default_rng(seed)
    return to_storage(rng.standard_normal((B, wl.d)), wl.dtype)


def make_small(d: int, V: int, c: int, B: int, seed: int, sigma_c: float = 1.0,
               sigma_n: float = 0.3, dtype: str = "f32") -> HeadData:
    """A small head of arbitrary shape built with the same recipe (V = b c)."""
    b = V // c
    assert b * c == V
    rng = np.random.default_rng(seed)
    M = rng.standard_normal((c, d)) * sigma_c
    noise = rng.standard_normal((V, d)) * sigma_n
    perm = rng.permutation(V)
    h = rng.standard_normal((B, d))
    lat = np.arange(V) // b
    E = to_storage((M[lat] + noise)[perm], dtype)
    wl = Workload(f"small_{d}_{V}_{c}", d=d, V=V, c=c, B=B, p=1, sigma_c=sigma_c,
                  sigma_n=sigma_n, dtype=dtype, e_pack=dtype, temperatures=(1.0,))
    return HeadData(wl=wl, E=E, h=to_storage(h, dtype), latent=lat[perm])


def make_unequal_clusters(latent: np.ndarray, c: int, seed: int, sigma: float = 0.5):
    """An unequal clustering of the V tokens into c clusters: the input of the equal- versus
    unequal-cluster ablation (FlashHead paper, Section 4.5, Table 6).

    Cluster sizes are drawn as max(1, rne(m exp(sigma z - sigma^2 / 2))), z ~ N(0, 1), m = V / c
    (a lognormal spread around the equal size), then single tokens are added to or taken from
    random clusters (never below 1) until they sum to V.  The tokens, ordered by latent label
    and then id, are cut into consecutive runs of those sizes, so a cluster holds tokens of one
    or a few neighbouring latent groups.  Returns (C2T [c][b_max] int32 with each row's tokens
    in ascending id followed by -1 padding, sizes [c] int64).
    """
    latent = np.asarray(latent)
    V = latent.size
    rng = np.random.default_rng(seed)
    m = V / c
    sizes = np.maximum(1, np.rint(m * np.exp(sigma * rng.standard_normal(c) - sigma * sigma / 2))).astype(np.int64)
    diff = int(V - sizes.sum())
    while diff != 0:
        k = int(rng.integers(c))
        if diff > 0:
            sizes[k] += 1
            diff -= 1
        elif sizes[k] > 1:
            sizes[k] -= 1
            diff += 1
    order = np.lexsort((np.arange(V), latent))
    C2T = np.full((c, int(sizes.max())), -1, dtype=np.int32)
    start = 0
    for k in range(c):
        C2T[k, :sizes[k]] = np.sort(order[start:start + sizes[k]])
        start += sizes[k]
    return C2T, sizes
