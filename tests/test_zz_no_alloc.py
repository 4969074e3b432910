"""flashhead_forward_noalloc (the static-scratch forward) against flashhead_forward.

Two calls in a row on one device share the library's scratch; the second, with a smaller head
and batch, must not see anything of the first.  Outputs must equal flashhead_forward's (with a
workspace of its own) bit for bit: the same kernels run on the same inputs.
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


def _head(gpu, d, b, c, B, seed):
    hd = workloads.make_small(d, b * c, c, B, seed=seed, sigma_c=1.0, sigma_n=0.5, dtype="bf16")
    C2T = H.latent_clusters(hd.latent, c)
    C = kmeans.centroids_from_c2t(ohead.decode(hd.E, "bf16"), C2T, "bf16")
    return DeviceHead(d, b * c, c, C, C2T, hd.E, "bf16", "bf16", "bf16", "bf16", device=gpu), to_device(hd.h, gpu)


def _both(dev, h, p, mode):
    B = h.shape[0]
    ref = dev.forward(h, p, mode=mode, tau=0.9, seed=7, step=3)
    got = dev.outputs(B, p)
    fh.flashhead_forward_noalloc(dev.desc(B), h, dev.C, dev.c2t, dev.tiles, dev.scales, p, mode, 0.9, 7, 3,
                                 fh.make_outputs(got["token"], got["probe_ids"], got["probe_logits"],
                                                 got["probe_tokens"]))
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(ref[k], got[k]), f"{k} differs from flashhead_forward"


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_noalloc_forward_twice_second_smaller(gpu, mode):
    big, hb = _head(gpu, 256, 16, 2000, 40, 31)          # batched: MFMA stage 1, masks, lists
    small, hs = _head(gpu, 128, 16, 300, 1, 32)          # B = 1: the fused selection + stage 2
    _both(big, hb, 60, mode)
    _both(small, hs, 9, mode)


def test_noalloc_forward_gemma_shape_then_smaller(gpu):
    wl, hd, C2T, C = H.load("gemma")
    dev = DeviceHead(wl.d, wl.V, wl.c, C, C2T, hd.E, wl.dtype, wl.dtype, wl.e_pack, wl.dtype, device=gpu)
    _both(dev, to_device(hd.h, gpu), wl.p, "greedy")
    small, hs = _head(gpu, 64, 8, 500, 3, 33)
    _both(small, hs, 5, "greedy")


def test_noalloc_rejects_a_workspace_beyond_the_scratch(gpu):
    desc = fh.make_desc(64, 1024, 32768 * 16, 32768)     # 64 x 32768 keys: 8 MiB
    assert fh.flashhead_workspace_bytes(desc, 256) > fh.NOALLOC_SCRATCH_BYTES
    out = fh.make_outputs(torch.empty(64, dtype=torch.int32, device=gpu))
    x = torch.empty(16, dtype=torch.uint8, device=gpu)
    with pytest.raises(fh.FlashHeadError) as ei:
        fh.flashhead_forward_noalloc(desc, x, x, x, x, None, 256, "greedy", 1.0, 0, 0, out)
    assert ei.value.status == fh.FH_ERR_UNSUPPORTED
