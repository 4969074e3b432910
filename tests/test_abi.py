"""The C ABI on the host: the library loads, exports what include/flashhead.h declares, and
rejects bad arguments before enqueuing anything (no GPU work is started by these tests)."""
from __future__ import annotations

import ctypes
import os
import subprocess

import pytest

from clustered_retrieval_lm_amd import flashhead as fh

FAKE = 0x10000          # a non-NULL pointer value; every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fh.LIB_PATH):
        from clustered_retrieval_lm_amd import build
        build.build()
    return fh.load_library()


def test_exports_every_declared_function(lib):
    names = fh.header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    syms = subprocess.run(["nm", "-D", "--defined-only", fh.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in syms.splitlines() if " T " in ln}
    assert set(names) <= exported
    assert all(not s.startswith("flashhead_") or s in names for s in exported), "undeclared export"


def test_version(lib):
    assert fh.flashhead_version().startswith("flashhead ")


def test_workspace_bytes(lib):
    d = fh.make_desc(1, 1152, 262144, 16384)
    n512 = fh.flashhead_workspace_bytes(d, 512)
    n1 = fh.flashhead_workspace_bytes(d, 1)
    assert n512 >= 16384 * 4 + 512 * 4 + 8 and n512 > n1
    assert n512 % 256 == 0
    d64 = fh.make_desc(64, 1024, 151936, 9496)
    assert fh.flashhead_workspace_bytes(d64, 256) >= 64 * 9496 * 4 + 9496 * 8 + 64 * 256 * 4
    assert fh.flashhead_dense_workspace_bytes(d) >= 8


def _ws(desc, p):
    n = ctypes.c_size_t(0)
    return fh.load_library().flashhead_workspace_bytes(ctypes.byref(desc) if desc is not None else None, p,
                                                       ctypes.byref(n))


@pytest.mark.parametrize("kw,status", [
    (dict(B=1, d=1152, V=262145, c=16384), fh.FH_ERR_SHAPE),          # c does not divide V
    (dict(B=0, d=1152, V=262144, c=16384), fh.FH_ERR_SHAPE),
    (dict(B=1, d=1150, V=262144, c=16384), fh.FH_ERR_SHAPE),          # d % 8
    (dict(B=1, d=1160, V=262144, c=16384, e_dtype="int4"), fh.FH_ERR_SHAPE),   # int4 needs d % 128
    (dict(B=1, d=1152, V=262144, c=16384, h_dtype=7), fh.FH_ERR_DTYPE),
    (dict(B=1, d=1152, V=262144, c=16384, c_dtype=7), fh.FH_ERR_DTYPE),
    (dict(B=1, d=1160, V=262144, c=16384, c_dtype=fh.FH_INT4_G128), fh.FH_ERR_SHAPE),  # int4 centroids: d % 128
    (dict(B=1, d=8192, V=262144, c=16384), fh.FH_ERR_UNSUPPORTED),    # bf16 rows limited to d <= 4096
    (dict(B=1, d=1152, V=65536 * 16, c=65536), fh.FH_ERR_UNSUPPORTED),  # c > 32768
    (dict(B=1, d=1152, V=512 * 300, c=300), fh.FH_ERR_UNSUPPORTED),   # b > 256
    (dict(B=70000, d=1152, V=262144, c=16384), fh.FH_ERR_UNSUPPORTED),
])
def test_desc_validation(lib, kw, status):
    args = dict(h_dtype="bf16", c_dtype="bf16", e_dtype="bf16")
    args.update(kw)
    d = fh.make_desc(args.pop("B"), args.pop("d"), args.pop("V"), args.pop("c"), **args)
    assert _ws(d, 4) == status
    assert fh.flashhead_last_error()


def test_null_and_reserved(lib):
    assert _ws(None, 4) == fh.FH_ERR_ARG
    d = fh.make_desc(1, 1152, 262144, 16384)
    d.reserved = 1
    assert _ws(d, 4) == fh.FH_ERR_ARG


def test_p_range(lib):
    d = fh.make_desc(1, 1152, 262144, 16384)
    assert _ws(d, 0) == fh.FH_ERR_ARG
    assert _ws(d, 16385) == fh.FH_ERR_ARG
    assert _ws(d, 16384) == fh.FH_OK


def _forward(desc, p=8, mode=0, tau=1.0, h=FAKE, C=FAKE, c2t=FAKE, tiles=FAKE, scales=None, ws=FAKE,
             ws_bytes=1 << 30, token=FAKE):
    out = fh.fh_outputs(token, None, None, None)
    return fh.load_library().flashhead_forward(ctypes.byref(desc), h, C, c2t, tiles, scales, p, mode, tau, 0, 0,
                                               ws, ws_bytes, ctypes.byref(out), None)


def test_forward_argument_checks(lib):
    d = fh.make_desc(1, 1152, 262144, 16384)
    assert _forward(d, mode=1, tau=0.0) == fh.FH_ERR_ARG
    assert _forward(d, mode=1, tau=float("nan")) == fh.FH_ERR_ARG
    assert _forward(d, mode=1, tau=-1.0) == fh.FH_ERR_ARG
    assert _forward(d, mode=5) == fh.FH_ERR_ARG
    assert _forward(d, h=None) == fh.FH_ERR_ARG
    assert _forward(d, C=None) == fh.FH_ERR_ARG
    assert _forward(d, c2t=None) == fh.FH_ERR_ARG
    assert _forward(d, token=None) == fh.FH_ERR_ARG
    assert _forward(d, ws=None) == fh.FH_ERR_WORKSPACE
    assert _forward(d, ws_bytes=100) == fh.FH_ERR_WORKSPACE
    assert "smaller than" in fh.flashhead_last_error()
    d4 = fh.make_desc(1, 3072, 128256, 8016, e_dtype="int4")
    assert _forward(d4, scales=None) == fh.FH_ERR_ARG        # int4 tiles need scales
    assert _forward(d4, p=0) == fh.FH_ERR_ARG


def test_stage_and_dense_argument_checks(lib):
    L = fh.load_library()
    d = fh.make_desc(1, 1152, 262144, 16384)
    assert L.flashhead_centroid_scores(ctypes.byref(d), None, FAKE, 0, 1.0, 0, 0, FAKE, 1 << 30, None, None) \
        == fh.FH_ERR_ARG
    assert L.flashhead_select_probes(ctypes.byref(d), 0, FAKE, 1 << 30, None, None) == fh.FH_ERR_ARG
    assert L.flashhead_select_probes(ctypes.byref(d), 8, FAKE, 10, None, None) == fh.FH_ERR_WORKSPACE
    out = fh.fh_outputs(None, None, None, None)
    assert L.flashhead_probe_logits(ctypes.byref(d), 8, FAKE, FAKE, FAKE, None, 0, 1.0, 0, 0, FAKE, 1 << 30,
                                    ctypes.byref(out), None) == fh.FH_ERR_ARG
    d4 = fh.make_desc(1, 3072, 128256, 8016, e_dtype="int4")
    d4s = fh.make_desc(1, 3080, 128256, 8016, e_dtype="int4")        # int4 rows need d % 128 == 0
    assert L.flashhead_dense_forward(ctypes.byref(d4s), FAKE, FAKE, 0, 1.0, 0, 0, FAKE, 1 << 20, FAKE, None, None) \
        == fh.FH_ERR_SHAPE
    assert L.flashhead_dense_forward(ctypes.byref(d4), FAKE, None, 0, 1.0, 0, 0, FAKE, 1 << 20, FAKE, None, None) \
        == fh.FH_ERR_ARG
    assert L.flashhead_dense_forward(ctypes.byref(d), FAKE, FAKE, 0, 1.0, 0, 0, FAKE, 0, FAKE, None, None) \
        == fh.FH_ERR_WORKSPACE
    assert L.flashhead_pack(ctypes.byref(d), 2, FAKE, FAKE, FAKE, None, None) == fh.FH_ERR_DTYPE
    assert L.flashhead_pack(ctypes.byref(d), 1, FAKE, FAKE, FAKE, FAKE, None) == fh.FH_ERR_ARG   # scales w/o int4
    assert L.flashhead_pack(ctypes.byref(d4), 1, FAKE, FAKE, FAKE, None, None) == fh.FH_ERR_ARG


def test_binding_raises(lib):
    with pytest.raises(fh.FlashHeadError) as ei:
        fh.flashhead_workspace_bytes(fh.make_desc(1, 1152, 262145, 16384), 4)
    assert ei.value.status == fh.FH_ERR_SHAPE


def _mc(desc, p=8, tau=1.0, n_sets=100, clip=1, h=FAKE, C=FAKE, c2t=FAKE, tiles=FAKE, scales=None, ws=FAKE,
        ws_bytes=1 << 34, out=FAKE):
    return fh.load_library().flashhead_mc_marginal(ctypes.byref(desc), h, C, c2t, tiles, scales, p, tau, 0, n_sets,
                                                   clip, ws, ws_bytes, out, None)


def test_mc_marginal_argument_checks(lib):
    d = fh.make_desc(1, 1152, 262144, 16384)
    need = fh.flashhead_mc_marginal_workspace_bytes(d)
    # the forward workspace at p = c, the logits of every token, and fp64 per-cluster state
    assert need >= fh.flashhead_workspace_bytes(d, 16384) + 262144 * 4 + 3 * 16384 * 8
    assert _mc(d, tau=0.0) == fh.FH_ERR_ARG
    assert _mc(d, tau=float("inf")) == fh.FH_ERR_ARG
    assert _mc(d, p=0) == fh.FH_ERR_ARG
    assert _mc(d, p=16385) == fh.FH_ERR_ARG
    assert _mc(d, n_sets=0) == fh.FH_ERR_ARG
    assert _mc(d, n_sets=1 << 31) == fh.FH_ERR_ARG
    assert _mc(d, clip=2) == fh.FH_ERR_ARG
    assert _mc(d, out=None) == fh.FH_ERR_ARG
    assert _mc(d, C=None) == fh.FH_ERR_ARG
    assert _mc(d, ws=None) == fh.FH_ERR_WORKSPACE
    assert _mc(d, ws_bytes=need - 1) == fh.FH_ERR_WORKSPACE
    d4 = fh.make_desc(1, 3072, 128256, 8016, e_dtype="int4")
    assert _mc(d4, scales=None) == fh.FH_ERR_ARG


def test_philox_words_argument_checks(lib):
    L = fh.load_library()
    assert L.flashhead_philox_words(1, 0, 0, 4, 0, 16, FAKE, None, None) == fh.FH_ERR_ARG       # stream 0..3
    assert L.flashhead_philox_words(1, 0, 0, 0, 0, -1, FAKE, None, None) == fh.FH_ERR_ARG       # count < 0
    assert L.flashhead_philox_words(1, 0, 0, 0, 0xFFFFFFFF, 2, FAKE, None, None) == fh.FH_ERR_ARG   # n past 2^32
    assert L.flashhead_philox_words(1, 0, 0, 0, 0, 16, None, None, None) == fh.FH_ERR_ARG      # no output
    assert L.flashhead_philox_words(1, 0, 0, 0, 5, 0, FAKE, None, None) == fh.FH_OK            # nothing to do
