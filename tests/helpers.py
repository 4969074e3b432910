"""Shared test machinery: workload loading and the GPU-vs-oracle comparison rules.

Comparison rules (FlashHead paper, Section 3.2, defines what is computed; the rounding
model is ours):
  * every GPU key / logit must lie within its rounding bound of the oracle's fp64 value;
  * probe sets must be equal unless the oracle's gap between the p-th and (p+1)-th key
    is within the two keys' bounds (the row is then "flagged" and only checked for
    validity: p distinct clusters, each within the bounds of the boundary);
  * tokens must be equal unless the probe set was flagged or the top-two token keys are
    within their bounds (then the GPU token must be one whose key is within the bounds
    of the maximum);
  * logits: |dz| <= 2e-2 for bf16 / int4 inputs, <= 1e-5 max(|z|, 1) for fp32.

Rounding bound of an fp32 dot product computed as a chain of L roundings (fused
multiply-adds, tree levels): |fl(s) - s| <= gamma_L * sum_j |h_j x_j|, gamma_L = L u / (1 - L u),
u = 2^-24 (Higham, "Accuracy and Stability of Numerical Algorithms", Sec. 3.1).  Each kernel
path's L follows from its accumulation order:
  row GEMV (16-byte chunks, 64 lanes): L = CH * EPC + 6   (per-lane FMA chain, 6 butterfly levels)
  B > 1 stage 2, bf16 rows and bf16 h:  L = 16 * CH + 6    (per-lane chain of 4 CH v_dot2c_f32_bf16, each
                                        counted as 4 roundings: its error, measured on the GPU, stays
                                        below 2.8 u (|p0| + |p1| + |acc|))
  int4 rows:                            L = 32 + CH + 7    (32-product chunk sum, scaled chain, tree)
  bf16 MFMA 16x16x32, K split 8 ways:   L = 6 * ceil(S / A) + log2(A) + 3, S = ceil(d / 256) K-steps per
                                        wave, A = 4 / 2 / 1 accumulators per tile when the batch spans
                                        one / two / more 16-row tiles; <= 6 roundings per MFMA, the tree
                                        over the A accumulators, a 3-level LDS tree over the 8 waves
The tests also assert that every observed error is within the bound, so a wrong L fails
loudly instead of hiding mismatches.
"""
from __future__ import annotations

import functools
import os

import numpy as np

import workloads
from oracle import head as ohead
from oracle import kmeans, philox

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U = 2.0 ** -24
EPC = {"f32": 4, "bf16": 8, "int4": 32}
ROW_BYTES = {"f32": 4.0, "bf16": 2.0, "int4": 0.5}


def gamma(L: int) -> float:
    return L * U / (1.0 - L * U)


def chunk_slots(fmt: str, d: int) -> int:
    cpr = int(d * ROW_BYTES[fmt]) // 16
    return (cpr + 63) // 64


def L_gemv(fmt: str, d: int) -> int:
    ch = chunk_slots(fmt, d)
    if fmt == "int4":
        return 32 + ch + 7
    return ch * EPC[fmt] + 6


def L_stage2(B: int, h_dtype: str, e_dtype: str, d: int) -> int:
    """Rounding depth of the stage-2 logits: the batched kernel dots bf16 rows with bf16 h by
    packed bf16 dot instructions, every other path by the row GEMV's FMA chain."""
    if B > 1 and h_dtype == "bf16" and e_dtype == "bf16":
        return 16 * chunk_slots("bf16", d) + 6
    return L_gemv(e_dtype, d)


def L_mfma(d: int, B: int = None) -> int:
    """Rounding depth of the batched MFMA product for a batch of B rows (None: the largest over B)."""
    npairs = -(-(-(-d // 32)) // 2)           # K-steps of 32 columns, handed to the waves in pairs
    steps = 2 * (-(-npairs // 8))              # steps of the busiest of the 8 waves
    levels = {1: 0, 2: 1, 4: 2}

    def depth(acc):
        return 6 * (-(-steps // acc)) + levels[acc] + 3
    if B is None:
        return max(depth(1), depth(2), depth(4))
    nt = 4 if B >= 64 else (B + 15) // 16
    return depth({1: 4, 2: 2}.get(nt, 1))


def L_stage1(B: int, h_dtype: str, c_dtype: str, d: int) -> int:
    if B > 1 and h_dtype == "bf16" and c_dtype == "bf16" and d % 32 == 0:
        return L_mfma(d, B)
    return L_gemv(c_dtype, d)


def key_bound(z: np.ndarray, A: np.ndarray, L: int, sample: bool, tau: float, G=None) -> np.ndarray:
    """Bound on |GPU key - exact key| for logits z with absolute sums A (0 for the -inf logit of
    an empty slot, which both sides report exactly)."""
    e = gamma(L) * A
    if not sample:
        return e
    fin = np.isfinite(z)
    x = np.where(fin, np.abs(z), 0.0) / tau
    g = np.where(fin, np.abs(G), 0.0)
    # z/tau rounded, G from two fp32 logs (taken as within 2^-20 (1 + |G|)), the sum rounded
    return np.where(fin, e / tau + U * x + 2.0 ** -20 * (1.0 + g) + U * (x + g) * 1.001 + 1e-30, 0.0)


@functools.lru_cache(maxsize=None)
def _c2t(name: str) -> np.ndarray:
    path = os.path.join(GOLDEN, f"clusters_{name}.npz")
    if not os.path.exists(path):
        import pytest
        pytest.skip(f"{path} not generated (tests/golden/make_clusterings.py)")
    return np.load(path)["C2T"]


def cluster_file(name: str) -> str:
    return {"int4_b16": "int4", "gemma_c4": "gemma"}.get(name, name)


def centroid_buffer(C, c_dtype: str) -> np.ndarray:
    """Stored centroids as the library takes them: f32 / bf16 arrays as they are; int4 as
    one byte buffer (nibbles [c][d/2], then from round_up(c d / 2, 256) the bf16 scales)."""
    if c_dtype != "int4":
        return C
    q, sc = C
    off = (q.size + 255) // 256 * 256
    buf = np.zeros(off + sc.size * 2, dtype=np.uint8)
    buf[:q.size] = q.reshape(-1)
    buf[off:] = np.ascontiguousarray(sc, dtype=np.uint16).reshape(-1).view(np.uint8)
    return buf


@functools.lru_cache(maxsize=4)
def load(name: str):
    """(workload, HeadData, C2T, centroids) with the oracle's clustering of the workload."""
    wl = workloads.WORKLOADS[name]
    hd = workloads.make_head(wl)
    C2T = _c2t(cluster_file(name))
    C = kmeans.centroids_from_c2t(ohead.decode(hd.E, wl.dtype), C2T, wl.c_dtype)
    return wl, hd, C2T, C


@functools.lru_cache(maxsize=8)
def oracle_tiles(name: str):
    wl, hd, C2T, _ = load(name)
    return ohead.pack_tiles(hd.E, wl.dtype, C2T, wl.e_pack)


def latent_clusters(latent: np.ndarray, c: int) -> np.ndarray:
    """The generator's latent partition as a balanced C2T (ascending ids per cluster).

    Small parity heads use it instead of a k-means run: the forward pass takes any
    balanced clustering, and this one is free to compute.
    """
    order = np.lexsort((np.arange(latent.size), latent))
    return order.reshape(c, -1).astype(np.int32)


class Report:
    def __init__(self):
        self.rows = 0
        self.flag_probe = 0
        self.flag_token = 0
        self.max_key_err_ratio = 0.0
        self.max_logit_err = 0.0

    def __str__(self):
        return (f"rows={self.rows} flagged_probe={self.flag_probe} flagged_token={self.flag_token} "
                f"max_key_err/bound={self.max_key_err_ratio:.3g} max_logit_err={self.max_logit_err:.3g}")

    def check_flag_rate(self) -> None:
        """Near ties are rare on these inputs: at most max(2, ceil(rows / 10)) rows may be flagged,
        so a regression that widens the bounds until most rows are flagged cannot pass.  (The
        largest expected rate, about 6 %, is the int4 head's batched stage 1 at d = 3072.)"""
        lim = flag_limit(self.rows)
        assert self.flag_probe <= lim, f"{self.flag_probe} of {self.rows} probe sets flagged (limit {lim})"
        assert self.flag_token <= lim, f"{self.flag_token} of {self.rows} tokens flagged (limit {lim})"


def flag_limit(rows: int) -> int:
    return max(2, -(-rows // 10))


def top_p_ids(keys: np.ndarray, p: int) -> np.ndarray:
    """Ids of the p largest keys (ties to the smaller id), ascending."""
    keys = np.asarray(keys, dtype=np.float64)
    ids = np.arange(keys.size)
    return np.sort(np.lexsort((ids, -keys))[:p])


def stage1_bounds(ref: ohead.HeadResult, r: int, L1: int, sample: bool, tau: float, seed: int, step: int):
    c = ref.s.shape[1]
    G1 = philox.gumbel(philox.uniform(seed, r, step, 0, np.arange(c))) if sample else None
    return key_bound(ref.s[r], ref.abss[r], L1, sample, tau, G1)


def stage2_bounds(ref: ohead.HeadResult, r: int, L2: int, sample: bool, tau: float, seed: int, step: int):
    flat_tok = ref.tokens[r].reshape(-1)
    G2 = philox.gumbel(philox.uniform(seed, r, step, 1, np.maximum(flat_tok, 0))) if sample else None
    return key_bound(ref.z[r].reshape(-1), ref.absz[r].reshape(-1), L2, sample, tau, G2)


def row_flags(ref: ohead.HeadResult, r: int, p: int, L1: int, L2: int, sample: bool, tau: float, seed: int,
              step: int):
    """(probe set flagged, token flagged) for row r: decided by the oracle's values and the rounding
    bounds alone, so the expected flag counts of a test can be computed without a GPU."""
    c = ref.s.shape[1]
    e1 = stage1_bounds(ref, r, L1, sample, tau, seed, step)
    order = ref.order1[r]
    fp = False
    if p < c:
        kp, kq = order[p - 1], order[p]
        fp = bool(ref.key1[r][kp] - ref.key1[r][kq] <= e1[kp] + e1[kq])
    if fp:
        return True, True
    flat_key = ref.key2[r].reshape(-1)
    e2 = stage2_bounds(ref, r, L2, sample, tau, seed, step)
    o2 = ref.order2[r]
    ft = bool(flat_key.size > 1 and np.isfinite(flat_key[o2[1]])
              and (flat_key[o2[0]] - flat_key[o2[1]] <= e2[o2[0]] + e2[o2[1]]))
    return False, ft


def compare_row(ref: ohead.HeadResult, r: int, got_ids: np.ndarray, got_z: np.ndarray, got_tok_ids: np.ndarray,
                got_token: int, p: int, L1: int, L2: int, sample: bool, tau: float, seed: int, step: int,
                fp32_inputs: bool, rep: Report, got_keys=None) -> None:
    """Check one row of a GPU forward against the oracle result `ref`."""
    rep.rows += 1
    c = ref.s.shape[1]
    e1 = stage1_bounds(ref, r, L1, sample, tau, seed, step)
    if got_keys is not None:
        err = np.abs(got_keys.astype(np.float64) - ref.key1[r])
        ratio = float(np.max(err / np.maximum(e1, 1e-300)))
        rep.max_key_err_ratio = max(rep.max_key_err_ratio, ratio)
        assert ratio <= 1.0, f"row {r}: stage-1 key error {err.max():.3g} exceeds its bound (ratio {ratio:.3g})"
    flagged, tok_flagged = row_flags(ref, r, p, L1, L2, sample, tau, seed, step)
    got_ids = np.asarray(got_ids, dtype=np.int64)
    assert np.all(np.diff(got_ids) > 0), f"row {r}: probe ids not strictly ascending"
    assert got_ids.size == p and got_ids.min() >= 0 and got_ids.max() < c
    if got_keys is not None:
        # the selection itself is exact: the kept set is the top p of the GPU's own keys
        assert np.array_equal(got_ids, top_p_ids(got_keys, p)), f"row {r}: probe set is not the top p of its keys"
    if not flagged:
        assert np.array_equal(got_ids, ref.probe_ids[r]), f"row {r}: probe set differs (unflagged)"
    else:
        rep.flag_probe += 1
        # every cluster that fewer than p others can outrank (within the bounds) is kept; every
        # cluster that at least p others surely outrank is not
        ub, lb = ref.key1[r] + e1, ref.key1[r] - e1
        can_outrank = ub.size - np.searchsorted(np.sort(ub), lb, side="left") - 1
        surely_above = lb.size - np.searchsorted(np.sort(lb), ub, side="right")
        must_keep = np.flatnonzero(can_outrank < p)
        must_drop = np.flatnonzero(surely_above >= p)
        assert np.all(np.isin(must_keep, got_ids)), f"row {r}: flagged probe set misses a cluster surely above"
        assert not np.any(np.isin(must_drop, got_ids)), f"row {r}: flagged probe set holds a cluster surely below"
    # logits of clusters both sides kept
    common, gi, oi = np.intersect1d(got_ids, ref.probe_ids[r], return_indices=True)
    zg = np.asarray(got_z, dtype=np.float64)[gi]
    zo = ref.z[r][oi]
    empty = ref.tokens[r][oi] < 0                 # empty slots of padded clusters: -inf on both sides
    assert np.all(zg[empty] == -np.inf), f"row {r}: an empty slot's logit is not -inf"
    zg, zo = np.where(empty, 0.0, zg), np.where(empty, 0.0, zo)
    dz = np.abs(zg - zo)
    rep.max_logit_err = max(rep.max_logit_err, float(dz.max()) if dz.size else 0.0)
    if fp32_inputs:
        assert np.all(dz <= 1e-5 * np.maximum(np.abs(zo), 1.0)), f"row {r}: fp32 logits out of tolerance"
    else:
        assert np.all(dz <= 2e-2), f"row {r}: logits differ by {dz.max():.3g} > 2e-2"
    ez = gamma(L2) * ref.absz[r][oi]
    assert np.all(dz <= ez + 1e-30), f"row {r}: logit error exceeds its rounding bound"
    assert np.array_equal(np.asarray(got_tok_ids)[gi], ref.tokens[r][oi]), f"row {r}: probe tokens differ"
    # the token is the maximum of the GPU's own gathered keys (exactly, for greedy keys)
    gz = np.asarray(got_z, dtype=np.float64).reshape(-1)
    gt = np.asarray(got_tok_ids, dtype=np.int64).reshape(-1)
    pos = np.flatnonzero(gt == int(got_token))
    assert pos.size == 1, f"row {r}: token {got_token} not among the gathered tokens"
    if not sample:
        assert int(got_token) == int(gt[np.lexsort((gt, -gz))[0]]), f"row {r}: token is not the largest gathered logit"
    else:
        g = philox.gumbel(philox.uniform(seed, r, step, 1, np.maximum(gt, 0)))
        x = gz / tau
        kk = np.where(gt >= 0, x + g, -np.inf)
        eb = np.where(gt >= 0, U * np.abs(np.where(gt >= 0, x, 0.0)) + 2.0 ** -20 * (1.0 + np.abs(g))
                      + U * (np.abs(np.where(gt >= 0, x, 0.0)) + np.abs(g)) * 1.001, 0.0)
        assert kk[pos[0]] + eb[pos[0]] >= np.max(kk - eb), f"row {r}: token is not the Gumbel-max of its logits"
    if flagged:
        rep.flag_token += 1
        return
    flat_key = ref.key2[r].reshape(-1)
    e2 = stage2_bounds(ref, r, L2, sample, tau, seed, step)
    o2 = ref.order2[r]
    if not tok_flagged:
        assert int(got_token) == int(ref.token[r]), f"row {r}: token {got_token} != oracle {ref.token[r]}"
    else:
        rep.flag_token += 1
        pos = np.flatnonzero(ref.tokens[r].reshape(-1) == int(got_token))
        assert pos.size == 1, f"row {r}: token {got_token} not among the oracle's gathered tokens"
        best = flat_key[o2[0]]
        assert flat_key[pos[0]] + e2[pos[0]] >= best - e2[o2[0]], f"row {r}: token far from the maximum"
