"""GPU parity of the FlashHead forward against the CPU oracle, through the C ABI.

Workloads: the tiny fp32 head, small heads with ragged shapes, and the full-size
Llama-3.2-1B / Gemma-3-1B / Qwen-3-0.6B / int4 head shapes (FlashHead paper, Section 4 and
Tables 3-7) with the oracle's balanced clusterings from tests/golden.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from clustered_retrieval_lm_amd import flashhead as fh
from clustered_retrieval_lm_amd.head import DeviceHead, to_device
from oracle import head as ohead
from oracle import kmeans

from . import helpers as H

pytestmark = pytest.mark.gpu


def _run_and_compare(dev: DeviceHead, hd_h: np.ndarray, h_dtype: str, C, C2T, tiles, p: int, mode: str,
                     tau: float, seed: int, step: int, fp32: bool, rep: H.Report, rows=None):
    B = hd_h.shape[0]
    h = to_device(hd_h, dev.device)
    out = dev.forward(h, p, mode=mode, tau=tau, seed=seed, step=step)
    # the staged entry points, with the stage-1 keys exposed
    ws = torch.empty_like(dev.workspace(B, p))
    desc = dev.desc(B)
    keys = torch.empty(B, dev.c, dtype=torch.float32, device=dev.device)
    fh.flashhead_centroid_scores(desc, h, dev.C, mode, tau, seed, step, ws, keys_out=keys)
    ids2 = torch.empty(B, p, dtype=torch.int32, device=dev.device)
    fh.flashhead_select_probes(desc, p, ws, ids2)
    o2 = dev.outputs(B, p)
    fh.flashhead_probe_logits(desc, p, h, dev.c2t, dev.tiles, dev.scales, mode, tau, seed, step, ws,
                              fh.make_outputs(o2["token"], None, o2["probe_logits"], o2["probe_tokens"]))
    # stage 1 then selection + stage 2 in one call (the two halves of flashhead_forward)
    o3 = dev.outputs(B, p)
    fh.flashhead_select_and_probe(desc, p, h, dev.c2t, dev.tiles, dev.scales, mode, tau, seed, step, ws,
                                  fh.make_outputs(o3["token"], o3["probe_ids"], o3["probe_logits"],
                                                  o3["probe_tokens"]))
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    for k, v in o3.items():
        assert np.array_equal(v.cpu().numpy(), got[k]), f"select_and_probe and forward differ in {k}"
    assert np.array_equal(ids2.cpu().numpy(), got["probe_ids"]), "staged and fused probe ids differ"
    assert np.array_equal(o2["token"].cpu().numpy(), got["token"]), "staged and fused tokens differ"
    assert np.array_equal(o2["probe_logits"].cpu().numpy(), got["probe_logits"])
    keys_np = keys.cpu().numpy()
    rows = range(B) if rows is None else rows
    ref = ohead.forward(hd_h, h_dtype, C, dev.c_dtype, C2T, tiles, p, mode=mode, tau=tau, seed=seed, step=step)
    L1 = H.L_stage1(B, h_dtype, dev.c_dtype, dev.d)
    L2 = H.L_stage2(B, h_dtype, dev.e_dtype, dev.d)
    for r in rows:
        H.compare_row(ref, r, got["probe_ids"][r], got["probe_logits"][r], got["probe_tokens"][r],
                      got["token"][r], p, L1, L2, mode == "sample", tau, seed, step, fp32, rep, got_keys=keys_np[r])
    return got


# ------------------------------------------------------------------ tiny head

def test_tiny_greedy_and_sample(gpu):
    wl, hd, C2T, C = H.load("tiny")
    dev = DeviceHead(wl.d, wl.V, wl.c, C, C2T, hd.E, "f32", "f32", "f32", "f32", device=gpu)
    tiles = H.oracle_tiles("tiny")
    rep = H.Report()
    _run_and_compare(dev, hd.h, "f32", C, C2T, tiles, wl.p, "greedy", 1.0, 0, 0, True, rep)
    for step in range(20):
        _run_and_compare(dev, hd.h, "f32", C, C2T, tiles, wl.p, "sample", 1.0, wl.sample_seed, step, True, rep)
    print(rep)
    rep.check_flag_rate()


# ------------------------------------------------------------------ small ragged heads

SMALL = [
    # d, b, c, B, p, dtype, e_dtype
    (136, 16, 1003, 1, 37, "bf16", "bf16"),     # ragged chunk slots, c % 4 != 0
    (136, 16, 1003, 3, 37, "bf16", "bf16"),     # B > 1 with a non-MFMA d (136 % 32 != 0)
    (256, 5, 777, 1, 1, "bf16", "bf16"),        # odd b, p = 1
    (256, 5, 777, 70, 9, "bf16", "bf16"),       # two mask words, MFMA with a ragged batch tile
    (384, 16, 512, 16, 512, "bf16", "bf16"),    # p = c
    (128, 1, 640, 2, 11, "bf16", "bf16"),       # b = 1
    (96, 16, 300, 1, 20, "f32", "f32"),         # fp32, ragged
    (96, 16, 300, 5, 20, "f32", "f32"),         # fp32 B > 1 (row GEMV per batch row)
    (512, 16, 400, 1, 33, "bf16", "int4"),      # int4 tiles
    (512, 16, 400, 16, 33, "bf16", "int4"),     # int4, batched
    (1024, 16, 600, 33, 25, "bf16", "int4"),    # int4, 2 chunk slots
]


@pytest.mark.parametrize("d,b,c,B,p,dt,et", SMALL)
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_small_heads(gpu, d, b, c, B, p, dt, et, mode):
    V = b * c
    hd = workloads.make_small(d, V, c, B, seed=1000 + d + c + B, sigma_c=1.0, sigma_n=0.5, dtype=dt)
    Ev = ohead.decode(hd.E, dt)
    C2T = H.latent_clusters(hd.latent, c)
    C = kmeans.centroids_from_c2t(Ev, C2T, dt)
    dev = DeviceHead(d, V, c, C, C2T, hd.E, dt, dt, et, dt, device=gpu)
    tiles = ohead.pack_tiles(hd.E, dt, C2T, et)
    rep = H.Report()
    tau = 0.7
    for step in (range(3) if mode == "sample" else [0]):
        _run_and_compare(dev, hd.h, dt, C, C2T, tiles, p, mode, tau, 5, step, dt == "f32", rep)
    print(rep)
    rep.check_flag_rate()


# ------------------------------------------------------------------ int4 centroids (stage 1)
# The paper's selective quantisation (Section 4.5, Table 5): stage 1 on int4 centroids,
# stage 2 on the bf16 tiles.

@pytest.mark.parametrize("B", [1, 5])
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_small_heads_int4_centroids(gpu, B, mode):
    d, b, c, p = 256, 16, 777, 40
    hd = workloads.make_small(d, b * c, c, B, seed=77 + B, sigma_c=1.0, sigma_n=0.5, dtype="bf16")
    C2T = H.latent_clusters(hd.latent, c)
    C = kmeans.centroids_from_c2t(ohead.decode(hd.E, "bf16"), C2T, "int4")
    dev = DeviceHead(d, b * c, c, H.centroid_buffer(C, "int4"), C2T, hd.E, "bf16", "int4", "bf16", "bf16",
                     device=gpu)
    tiles = ohead.pack_tiles(hd.E, "bf16", C2T, "bf16")
    rep = H.Report()
    for step in (range(3) if mode == "sample" else [0]):
        _run_and_compare(dev, hd.h, "bf16", C, C2T, tiles, p, mode, 0.9, 5, step, False, rep)
    print(rep)
    rep.check_flag_rate()


# ------------------------------------------------------------------ full-size heads

FULL = [("llama", "greedy", 1.0), ("gemma", "greedy", 1.0), ("gemma", "sample", 1.0),
        ("qwen", "greedy", 1.0), ("qwen", "sample", 0.8), ("int4", "greedy", 1.0), ("int4", "sample", 1.0),
        ("int4_b16", "greedy", 1.0), ("int4_b16", "sample", 1.0), ("gemma_c4", "greedy", 1.0),
        ("gemma_c4", "sample", 1.0)]


@pytest.mark.parametrize("name,mode,tau", FULL)
def test_full_size(gpu, name, mode, tau):
    wl, hd, C2T, C = H.load(name)
    dev = DeviceHead(wl.d, wl.V, wl.c, H.centroid_buffer(C, wl.c_dtype), C2T, hd.E, wl.dtype, wl.c_dtype, wl.e_pack,
                     wl.dtype, device=gpu)
    tiles = H.oracle_tiles(name)
    rep = H.Report()
    steps = [0] if mode == "greedy" else [0, 1, 7, 123, 999]
    for step in steps:
        _run_and_compare(dev, hd.h, wl.dtype, C, C2T, tiles, wl.p, mode, tau, wl.sample_seed, step, False, rep)
    print(name, mode, rep)
    rep.check_flag_rate()


# ------------------------------------------------------------------ workspace reuse (B > 1)

@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_batched_selections_in_a_row_on_one_workspace(gpu, mode):
    """Two selections with different p on one workspace and no stage-1 call between them: the
    second one's outputs equal a forward at that p on a fresh workspace (the per-cluster state the
    batched stage 2 reads is the second selection's alone)."""
    d, b, c, B = 256, 16, 777, 70
    hd = workloads.make_small(d, b * c, c, B, seed=4242, sigma_c=1.0, sigma_n=0.5, dtype="bf16")
    C2T = H.latent_clusters(hd.latent, c)
    C = kmeans.centroids_from_c2t(ohead.decode(hd.E, "bf16"), C2T, "bf16")
    dev = DeviceHead(d, b * c, c, C, C2T, hd.E, "bf16", "bf16", "bf16", "bf16", device=gpu)
    h = to_device(hd.h, gpu)
    desc = dev.desc(B)
    ws = torch.empty(fh.flashhead_workspace_bytes(desc, 40), dtype=torch.uint8, device=gpu)
    fh.flashhead_centroid_scores(desc, h, dev.C, mode, 0.9, 3, 1, ws)
    wide = torch.empty(B, 40, dtype=torch.int32, device=gpu)
    fh.flashhead_select_probes(desc, 40, ws, wide)            # keeps 40 clusters per row ...
    for p in (9, 33):                                          # ... then fewer, on the same state
        o = dev.outputs(B, p)
        fh.flashhead_select_and_probe(desc, p, h, dev.c2t, dev.tiles, None, mode, 0.9, 3, 1, ws,
                                      fh.make_outputs(o["token"], o["probe_ids"], o["probe_logits"],
                                                      o["probe_tokens"]))
        fresh = dev.forward(h, p, mode=mode, tau=0.9, seed=3, step=1,
                            workspace=torch.empty(fh.flashhead_workspace_bytes(desc, p), dtype=torch.uint8,
                                                  device=gpu))
        torch.cuda.synchronize()
        for k in o:
            assert torch.equal(o[k], fresh[k]), f"p={p}: {k} differs after an earlier selection"
