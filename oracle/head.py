"""Dense head, tile packing and the FlashHead forward pass (oracle side, fp64).

The FlashHead paper, Section 3 ("Methodology"): the dense head computes the
logits z = E h over all v tokens and takes t = argmax z (greedy) or samples
t ~ Categorical(softmax(z / tau)).  FlashHead (Section 3.2, "Token retrieval
from Hidden Vector") instead scores the c centroids, C h, keeps p clusters --
the top p centroid logits for greedy decoding, or p clusters drawn without
replacement from the softmax of the centroid logits for sampling -- gathers the
tokens of those clusters through the dense cluster-to-token map C2T[c][b]
(Section 3.2, "Complexity"), computes their logits and takes the argmax, or
samples a token from the softmax of those logits.

Readings fixed here (the page is silent on them):
  * sampling without replacement is realised by Gumbel-top-p: the p largest
    keys s_k / tau + G_k, G_k = gumbel(U(seed, row, step, stream 0, n = k)),
    which is distributed exactly as successive draws without replacement;
  * the token sample is Gumbel-max over the gathered tokens with keys
    z_t / tau + gumbel(U(seed, row, step, stream 1, n = t)), t the vocabulary id;
  * tau applies to both stages;
  * ties: the larger key wins, then the smaller cluster id (probe selection)
    or the smaller vocabulary id (token);
  * probe_ids are reported in ascending cluster id, probe logits in that order;
  * unequal clusters (the ablation of Sections 3.1 and 4.5) keep the dense C2T padded to the
    largest cluster: an entry -1 is an empty slot, which gathers nothing -- its logit is
    reported as -inf and its token as -1, and it is never chosen.

All arithmetic is fp64 on exactly decoded inputs: products of bf16 / fp32 /
int4-dequantised values are exact in fp64.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import codecs, philox


def decode(x, dtype: str) -> np.ndarray:
    """Exact float64 values of stored f32 / bf16 arrays, or of int4 rows given as the pair
    (nibbles uint8 [..][d/2], bf16 scale bits [..][d/128])."""
    if dtype == "f32":
        return codecs.f32_to_f64(x)
    if dtype == "bf16":
        return codecs.bf16_to_f64(x)
    if dtype == "int4":
        q, sc = x
        return codecs.int4_dequantize(q, sc)
    raise ValueError(dtype)


# --------------------------------------------------------------------------- packing

@dataclasses.dataclass
class PackedTiles:
    """Cluster-major token embeddings: the rows of cluster k are contiguous."""
    dtype: str              # "f32" | "bf16" | "int4"
    data: np.ndarray        # f32: float32[c][b][d]; bf16: uint16[c][b][d]; int4: uint8[c][b][d/2]
    scales: np.ndarray = None   # int4 only: uint16 bf16 bits [c][b][d/128]

    def values(self, ks=None) -> np.ndarray:
        """Exact float64 values of the tiles (all, or the clusters in ks)."""
        data = self.data if ks is None else self.data[ks]
        if self.dtype == "int4":
            sc = self.scales if ks is None else self.scales[ks]
            return codecs.int4_dequantize(data, sc)
        return decode(data, self.dtype)


def pack_tiles(E: np.ndarray, e_dtype: str, C2T: np.ndarray, dst: str) -> PackedTiles:
    """Gather E's rows into cluster-major tiles, optionally quantised to int4; an empty slot
    (C2T entry -1) gets a zero row."""
    C2T = np.asarray(C2T, dtype=np.int64)
    rows = np.asarray(E)[np.maximum(C2T, 0)]                   # [c][b][d]
    rows[C2T < 0] = 0
    if dst == e_dtype:
        return PackedTiles(dst, np.ascontiguousarray(rows))
    vals = decode(rows, e_dtype)
    if dst == "int4":
        q, s = codecs.int4_quantize(vals)
        return PackedTiles("int4", q, s)
    if dst == "bf16":
        return PackedTiles("bf16", codecs.round_to_bf16(vals))
    if dst == "f32":
        return PackedTiles("f32", codecs.round_to_f32(vals))
    raise ValueError(dst)


# --------------------------------------------------------------------------- dense head

@dataclasses.dataclass
class DenseResult:
    z: np.ndarray        # [B][V] fp64 logits
    absz: np.ndarray     # [B][V] sum_j |h_j e_tj| (for rounding bounds)
    key: np.ndarray      # [B][V] keys the token is chosen by
    token: np.ndarray    # [B] int64


def dense_forward(h: np.ndarray, h_dtype: str, E: np.ndarray, e_dtype: str, mode: str = "greedy",
                  tau: float = 1.0, seed: int = 0, step: int = 0) -> DenseResult:
    H = decode(h, h_dtype)
    Ev = decode(E, e_dtype)
    z = H @ Ev.T
    absz = np.abs(H) @ np.abs(Ev).T
    B, V = z.shape
    key = np.empty_like(z)
    tok = np.empty(B, dtype=np.int64)
    ids = np.arange(V)
    for r in range(B):
        if mode == "greedy":
            key[r] = z[r]
        else:
            key[r] = z[r] / tau + philox.gumbel(philox.uniform(seed, r, step, 1, ids))
        tok[r] = ids[np.lexsort((ids, -key[r]))[0]]
    return DenseResult(z, absz, key, tok)


# --------------------------------------------------------------------------- FlashHead

@dataclasses.dataclass
class HeadResult:
    s: np.ndarray             # [B][c] centroid logits
    abss: np.ndarray          # [B][c] sum_j |h_j C_kj|
    key1: np.ndarray          # [B][c] probe-selection keys
    order1: np.ndarray        # [B][c] clusters by (key1 desc, id asc)
    probe_ids: np.ndarray     # [B][p] selected clusters, ascending id
    z: np.ndarray             # [B][p][b] logits of the gathered tokens
    absz: np.ndarray          # [B][p][b]
    tokens: np.ndarray        # [B][p][b] vocabulary ids of the gathered tokens
    key2: np.ndarray          # [B][p][b] token keys
    order2: np.ndarray        # [B][p*b] flat positions by (key2 desc, token id asc)
    token: np.ndarray         # [B]


def forward(h: np.ndarray, h_dtype: str, C: np.ndarray, c_dtype: str, C2T: np.ndarray,
            tiles: PackedTiles, p: int, mode: str = "greedy", tau: float = 1.0, seed: int = 0,
            step: int = 0) -> HeadResult:
    H = decode(h, h_dtype)
    Cv = decode(C, c_dtype)
    C2T = np.asarray(C2T, dtype=np.int64)
    c, b = C2T.shape
    B = H.shape[0]
    if not 1 <= p <= c:
        raise ValueError("need 1 <= p <= c")
    # stage 1: centroid logits C h
    s = H @ Cv.T
    abss = np.abs(H) @ np.abs(Cv).T
    ks = np.arange(c)
    key1 = np.empty_like(s)
    order1 = np.empty((B, c), dtype=np.int64)
    probe = np.empty((B, p), dtype=np.int64)
    z = np.empty((B, p, b))
    absz = np.empty((B, p, b))
    toks = np.empty((B, p, b), dtype=np.int64)
    key2 = np.empty((B, p, b))
    order2 = np.empty((B, p * b), dtype=np.int64)
    token = np.empty(B, dtype=np.int64)
    for r in range(B):
        if mode == "greedy":
            key1[r] = s[r]
        else:
            key1[r] = s[r] / tau + philox.gumbel(philox.uniform(seed, r, step, 0, ks))
        order1[r] = np.lexsort((ks, -key1[r]))
        probe[r] = np.sort(order1[r][:p])
        # stage 2: logits of the gathered tokens (empty slots of padded clusters gather nothing)
        T = tiles.values(probe[r])                             # [p][b][d]
        toks[r] = C2T[probe[r]]
        real = toks[r] >= 0
        z[r] = np.where(real, T @ H[r], -np.inf)
        absz[r] = np.where(real, np.abs(T) @ np.abs(H[r]), 0.0)
        if mode == "greedy":
            key2[r] = z[r]
        else:
            key2[r] = -np.inf
            key2[r][real] = z[r][real] / tau + philox.gumbel(philox.uniform(seed, r, step, 1, toks[r][real]))
        flat_t = toks[r].reshape(-1)
        order2[r] = np.lexsort((flat_t, -key2[r].reshape(-1)))
        token[r] = flat_t[order2[r][0]]
    return HeadResult(s, abss, key1, order1, probe, z, absz, toks, key2, order2, token)
