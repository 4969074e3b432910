"""GPU parity of unequal clusters: the padded dense C2T of the FlashHead paper's Section 3.1 (when
clusters are not equalised, C2T is sized by the largest cluster and the rows of smaller ones are
padded) and the ablation of Section 4.5 (Table 6).

The head is given to the library with b = the largest cluster size and C2T entries -1 in the
empty slots: flashhead_pack writes zero rows there and checks that the other entries are the
tokens 0 .. V-1 once each, flashhead_centroids averages the members only, and the forward path
never chooses an empty slot (reported as token -1 with logit -inf).  Everything is compared
with the oracle's padded forward.
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

CASES = [
    # d, V, c, B, p, tile dtype
    (256, 4000, 250, 1, 9, "bf16"),
    (256, 4000, 250, 5, 9, "bf16"),        # batched: MFMA stage 1, row masks, the kept list
    (512, 6400, 400, 1, 33, "int4"),
    (512, 6400, 400, 16, 33, "int4"),
    (96, 2400, 300, 1, 20, "f32"),
]


def _padded_head(gpu, d, V, c, B, et, seed):
    dt = "f32" if et == "f32" else "bf16"
    hd = workloads.make_small(d, V, c, B, seed=seed, sigma_c=1.0, sigma_n=0.5, dtype=dt)
    C2T, sizes = workloads.make_unequal_clusters(hd.latent, c, seed=seed + 1)
    slots = c * C2T.shape[1]
    dev = DeviceHead.from_clusters(d, slots, c, C2T, hd.E, dt, dt, et, dt, device=gpu)
    return hd, C2T, sizes, dev, dt


@pytest.mark.parametrize("d,V,c,B,p,et", CASES)
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_padded_clusters_match_the_oracle(gpu, d, V, c, B, p, et, mode):
    hd, C2T, sizes, dev, dt = _padded_head(gpu, d, V, c, B, et, seed=700 + d + c + B)
    assert sizes.max() > 2 * sizes.min()                       # really unequal
    Ev = ohead.decode(hd.E, dt)
    C = kmeans.centroids_from_c2t(Ev, C2T, dt)
    got_C = dev.C.cpu().numpy().view(np.uint16 if dt == "bf16" else np.float32).reshape(c, d)
    assert np.array_equal(got_C, C), "centroids of padded clusters differ from the member means"
    tiles = ohead.pack_tiles(hd.E, dt, C2T, et)
    h = to_device(hd.h, gpu)
    rep = H.Report()
    L1 = H.L_stage1(B, dt, dt, d)
    L2 = H.L_stage2(B, dt, et, d)
    for step in ([0] if mode == "greedy" else [0, 1, 2]):
        out = dev.forward(h, p, mode=mode, tau=0.8, seed=3, step=step)
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy() for k, v in out.items()}
        ref = ohead.forward(hd.h, dt, C, dt, C2T, tiles, p, mode=mode, tau=0.8, seed=3, step=step)
        for r in range(B):
            H.compare_row(ref, r, got["probe_ids"][r], got["probe_logits"][r], got["probe_tokens"][r], got["token"][r],
                          p, L1, L2, mode == "sample", 0.8, 3, step, dt == "f32", rep)
    print(rep)
    rep.check_flag_rate()




def test_pack_padded_tiles_bit_exact(gpu):
    hd, C2T, sizes, dev, dt = _padded_head(gpu, 128, 3000, 200, 1, "bf16", seed=9)
    ref = ohead.pack_tiles(hd.E, dt, C2T, "bf16")
    assert np.array_equal(dev.tiles.cpu().numpy(), np.ascontiguousarray(ref.data).view(np.uint8).reshape(-1))


@pytest.mark.parametrize("bad", ["duplicate", "gap", "beyond"])
def test_pack_rejects_a_malformed_padded_c2t(gpu, bad):
    d, c, b = 64, 10, 4
    C2T = np.full((c, b), -1, dtype=np.int32)
    C2T[:, :3] = np.arange(c * 3, dtype=np.int32).reshape(c, 3)   # 30 tokens, one empty slot each
    if bad == "duplicate":
        C2T[0, 3] = 7
    elif bad == "gap":
        C2T[0, 0] = -1                                              # token 0 missing
    else:
        C2T[0, 3] = 35                                              # 31 tokens, but 30 missing
    E = torch.zeros(c * b * d, dtype=torch.float32, device=gpu)
    tiles = torch.empty(c * b * d * 4, dtype=torch.uint8, device=gpu)
    with pytest.raises(fh.FlashHeadError) as ei:
        fh.flashhead_pack(fh.make_desc(1, d, c * b, c, "f32", "f32", "f32"), "f32", E, to_device(C2T, gpu), tiles)
    assert ei.value.status == fh.FH_ERR_ARG
