"""Device-resident FlashHead: uploads a clustered head once and calls the C ABI.

Holds the centroids, the cluster-to-token map, the packed tiles (made on the GPU by
flashhead_pack), a workspace and output buffers, all as torch tensors used purely as
device memory.  Every step of the head runs in libflashhead.so.
"""
from __future__ import annotations

import numpy as np
import torch

from . import flashhead as fh

_ELEM = {"f32": 4, "bf16": 2}


def to_device(a, device="cuda") -> torch.Tensor:
    """Copy a numpy array to the device bit for bit (bf16 bit patterns stay int16)."""
    if isinstance(a, torch.Tensor):
        return a.to(device)
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(device)


class DeviceHead:
    def __init__(self, d: int, V: int, c: int, centroids: np.ndarray, c2t: np.ndarray, E: np.ndarray,
                 e_src: str, c_dtype: str, e_dtype: str, h_dtype: str, device="cuda", keep_dense=False,
                 stream=None):
        self.d, self.V, self.c, self.b = d, V, c, V // c
        self.c_dtype, self.e_dtype, self.h_dtype, self.e_src = c_dtype, e_dtype, h_dtype, e_src
        self.device = device
        self.C = to_device(centroids, device)
        self.c2t = c2t.to(device) if isinstance(c2t, torch.Tensor) else to_device(np.asarray(c2t, np.int32), device)
        Ed = to_device(E, device)
        rows = c * self.b
        if e_dtype == "int4":
            self.tiles = torch.empty(rows * d // 2, dtype=torch.uint8, device=device)
            self.scales = torch.empty(rows * (d // 128), dtype=torch.int16, device=device)
        else:
            self.tiles = torch.empty(rows * d * _ELEM[e_dtype], dtype=torch.uint8, device=device)
            self.scales = None
        fh.flashhead_pack(self.desc(1), e_src, Ed, self.c2t, self.tiles, self.scales, stream=stream)
        self.E = Ed if keep_dense else None
        self._ws = {}

    @classmethod
    def from_clusters(cls, d: int, V: int, c: int, c2t: np.ndarray, E: np.ndarray, e_src: str, c_dtype: str,
                      e_dtype: str, h_dtype: str, device="cuda", keep_dense=False, unit=False, stream=None):
        """Build the head from a clustering alone: centroids computed on the GPU."""
        Ed = to_device(E, device)
        c2t_d = to_device(np.asarray(c2t, dtype=np.int32), device)
        desc = fh.make_desc(1, d, V, c, h_dtype, c_dtype, e_dtype)
        cent = torch.empty(fh.flashhead_centroids_bytes(desc), dtype=torch.uint8, device=device)
        fh.flashhead_centroids(desc, e_src, Ed, c2t_d, cent, unit=unit, stream=stream)
        return cls(d, V, c, cent, c2t_d, Ed, e_src, c_dtype, e_dtype, h_dtype, device, keep_dense, stream)

    def desc(self, B: int, e_dtype=None) -> fh.fh_desc:
        return fh.make_desc(B, self.d, self.V, self.c, self.h_dtype, self.c_dtype, e_dtype or self.e_dtype)

    def workspace(self, B: int, p: int) -> torch.Tensor:
        key = (B, p)
        if key not in self._ws:
            n = fh.flashhead_workspace_bytes(self.desc(B), p)
            self._ws[key] = torch.empty(n, dtype=torch.uint8, device=self.device)
        return self._ws[key]

    def outputs(self, B: int, p: int, probes=True) -> dict:
        o = {"token": torch.empty(B, dtype=torch.int32, device=self.device)}
        if probes:
            o["probe_ids"] = torch.empty(B, p, dtype=torch.int32, device=self.device)
            o["probe_logits"] = torch.empty(B, p, self.b, dtype=torch.float32, device=self.device)
            o["probe_tokens"] = torch.empty(B, p, self.b, dtype=torch.int32, device=self.device)
        return o

    def forward(self, h: torch.Tensor, p: int, mode="greedy", tau=1.0, seed=0, step=0, out=None,
                probes=True, stream=None, workspace=None) -> dict:
        B = h.shape[0]
        o = out if out is not None else self.outputs(B, p, probes)
        ws = workspace if workspace is not None else self.workspace(B, p)
        fo = fh.make_outputs(o["token"], o.get("probe_ids"), o.get("probe_logits"), o.get("probe_tokens"))
        fh.flashhead_forward(self.desc(B), h, self.C, self.c2t, self.tiles, self.scales, p, mode, tau, seed, step,
                             ws, fo, stream=stream)
        return o

    def mc_marginal(self, h: torch.Tensor, p: int, tau=1.0, seed=0, n_sets=10000, clip=True, out=None,
                    stream=None, workspace=None) -> torch.Tensor:
        """Monte-Carlo estimate of the sampler's distribution, float64 [B][V] by vocabulary id."""
        B = h.shape[0]
        desc = self.desc(B)
        ws = workspace
        if ws is None:
            ws = torch.empty(fh.flashhead_mc_marginal_workspace_bytes(desc), dtype=torch.uint8, device=self.device)
        o = out if out is not None else torch.empty(B, self.V, dtype=torch.float64, device=self.device)
        fh.flashhead_mc_marginal(desc, h, self.C, self.c2t, self.tiles, self.scales, p, tau, seed, n_sets, clip, ws,
                                 o, stream=stream)
        return o

    def dense(self, h: torch.Tensor, mode="greedy", tau=1.0, seed=0, step=0, logits=False, stream=None,
              token=None, workspace=None) -> dict:
        assert self.E is not None, "constructed without keep_dense"
        B = h.shape[0]
        desc = self.desc(B, e_dtype=self.e_src)
        ws = workspace
        if ws is None:
            ws = torch.empty(fh.flashhead_dense_workspace_bytes(desc), dtype=torch.uint8, device=self.device)
        tok = token if token is not None else torch.empty(B, dtype=torch.int32, device=self.device)
        lg = torch.empty(B, self.V, dtype=torch.float32, device=self.device) if logits else None
        fh.flashhead_dense_forward(desc, h, self.E, mode, tau, seed, step, ws, tok, lg, stream=stream)
        return {"token": tok, "logits": lg}
