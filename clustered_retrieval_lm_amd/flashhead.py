"""ctypes binding of libflashhead.so (declarations in include/flashhead.h).

Argument marshalling only: every function here forwards to the C entry point of the
same name.  Device buffers are torch tensors on the GPU (their data_ptr() is passed),
the stream defaults to torch's current stream.  A non-FH_OK status raises
FlashHeadError carrying the status and flashhead_last_error().  There is no fallback:
if the library is missing the import of a function raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libflashhead.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "flashhead.h")

FH_OK, FH_ERR_ARG, FH_ERR_SHAPE, FH_ERR_DTYPE, FH_ERR_UNSUPPORTED, FH_ERR_WORKSPACE, FH_ERR_HIP = range(7)
FH_F32, FH_BF16, FH_INT4_G128 = 0, 1, 2
FH_GREEDY, FH_SAMPLE = 0, 1
STATUS_NAMES = {0: "FH_OK", 1: "FH_ERR_ARG", 2: "FH_ERR_SHAPE", 3: "FH_ERR_DTYPE",
                4: "FH_ERR_UNSUPPORTED", 5: "FH_ERR_WORKSPACE", 6: "FH_ERR_HIP"}
DTYPES = {"f32": FH_F32, "bf16": FH_BF16, "int4": FH_INT4_G128}
MODES = {"greedy": FH_GREEDY, "sample": FH_SAMPLE}


class FlashHeadError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class fh_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("d", ctypes.c_int64), ("V", ctypes.c_int64), ("c", ctypes.c_int64),
                ("h_dtype", ctypes.c_int32), ("c_dtype", ctypes.c_int32), ("e_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class fh_outputs(ctypes.Structure):
    _fields_ = [("token", ctypes.c_void_p), ("probe_ids", ctypes.c_void_p),
                ("probe_logits", ctypes.c_void_p), ("probe_tokens", ctypes.c_void_p)]


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("FLASHHEAD_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(f"{p} not built: run __graft_entry__.build() or "
                                "python -m clustered_retrieval_lm_amd.build")
    lib = ctypes.CDLL(p)
    vp, i32, i64, u64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                  ctypes.c_float, ctypes.c_size_t)
    D = ctypes.POINTER(fh_desc)
    O = ctypes.POINTER(fh_outputs)
    sigs = {
        "flashhead_version": ([], ctypes.c_char_p),
        "flashhead_last_error": ([], ctypes.c_char_p),
        "flashhead_workspace_bytes": ([D, i64, ctypes.POINTER(sz)], ctypes.c_int),
        "flashhead_pack": ([D, i32, vp, vp, vp, vp, vp], ctypes.c_int),
        "flashhead_centroids": ([D, i32, vp, vp, i32, vp, vp], ctypes.c_int),
        "flashhead_centroids_bytes": ([D, ctypes.POINTER(sz)], ctypes.c_int),
        "flashhead_build_clusters_workspace_bytes": ([D, i32, ctypes.POINTER(sz)], ctypes.c_int),
        "flashhead_build_clusters": ([D, i32, vp, i32, u64, i32, vp, vp, vp, sz, vp], ctypes.c_int),
        "flashhead_centroid_scores": ([D, vp, vp, i32, f32, u64, u64, vp, sz, vp, vp], ctypes.c_int),
        "flashhead_select_probes": ([D, i64, vp, sz, vp, vp], ctypes.c_int),
        "flashhead_probe_logits": ([D, i64, vp, vp, vp, vp, i32, f32, u64, u64, vp, sz, O, vp], ctypes.c_int),
        "flashhead_select_and_probe": ([D, i64, vp, vp, vp, vp, i32, f32, u64, u64, vp, sz, O, vp], ctypes.c_int),
        "flashhead_forward": ([D, vp, vp, vp, vp, vp, i64, i32, f32, u64, u64, vp, sz, O, vp], ctypes.c_int),
        "flashhead_mc_marginal_workspace_bytes": ([D, ctypes.POINTER(sz)], ctypes.c_int),
        "flashhead_mc_marginal": ([D, vp, vp, vp, vp, vp, i64, f32, u64, i64, i32, vp, sz, vp, vp], ctypes.c_int),
        "flashhead_dense_workspace_bytes": ([D, ctypes.POINTER(sz)], ctypes.c_int),
        "flashhead_dense_forward": ([D, vp, vp, i32, f32, u64, u64, vp, sz, vp, vp, vp], ctypes.c_int),
        "flashhead_forward_noalloc": ([D, vp, vp, vp, vp, vp, i64, i32, f32, u64, u64, O, vp], ctypes.c_int),
        "flashhead_philox_words": ([u64, ctypes.c_uint32, u64, ctypes.c_uint32, ctypes.c_uint32, i64, vp, vp, vp],
                                   ctypes.c_int),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


def header_functions(header: str = HEADER) -> list:
    """Names of the functions include/flashhead.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flashhead_\w+)\s*\(", text)))


# ------------------------------------------------------------------ marshalling helpers

def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int) -> None:
    if status != FH_OK:
        msg = load_library().flashhead_last_error().decode()
        raise FlashHeadError(status, msg)


def make_desc(B: int, d: int, V: int, c: int, h_dtype="bf16", c_dtype="bf16", e_dtype="bf16") -> fh_desc:
    conv = lambda x: DTYPES[x] if isinstance(x, str) else int(x)  # noqa: E731
    return fh_desc(B, d, V, c, conv(h_dtype), conv(c_dtype), conv(e_dtype), 0)


def make_outputs(token, probe_ids=None, probe_logits=None, probe_tokens=None) -> fh_outputs:
    return fh_outputs(_ptr(token), _ptr(probe_ids), _ptr(probe_logits), _ptr(probe_tokens))


def _mode(mode) -> int:
    return MODES[mode] if isinstance(mode, str) else int(mode)


# ------------------------------------------------------------------ C entry points

def flashhead_version() -> str:
    return load_library().flashhead_version().decode()


def flashhead_last_error() -> str:
    return load_library().flashhead_last_error().decode()


def flashhead_workspace_bytes(desc: fh_desc, p: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().flashhead_workspace_bytes(ctypes.byref(desc), p, ctypes.byref(n)))
    return n.value


def flashhead_dense_workspace_bytes(desc: fh_desc) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().flashhead_dense_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def flashhead_pack(desc: fh_desc, src_dtype, E, cluster_tokens, E_tiles, E_scales=None, stream=None) -> None:
    src = DTYPES[src_dtype] if isinstance(src_dtype, str) else int(src_dtype)
    _check(load_library().flashhead_pack(ctypes.byref(desc), src, _ptr(E), _ptr(cluster_tokens), _ptr(E_tiles),
                                         _ptr(E_scales), _stream(stream)))


def flashhead_centroids(desc: fh_desc, src_dtype, E, cluster_tokens, centroids, unit=False, stream=None) -> None:
    src = DTYPES[src_dtype] if isinstance(src_dtype, str) else int(src_dtype)
    _check(load_library().flashhead_centroids(ctypes.byref(desc), src, _ptr(E), _ptr(cluster_tokens), int(bool(unit)),
                                              _ptr(centroids), _stream(stream)))


def flashhead_centroids_bytes(desc: fh_desc) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().flashhead_centroids_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def flashhead_build_clusters_workspace_bytes(desc: fh_desc, src_dtype) -> int:
    src = DTYPES[src_dtype] if isinstance(src_dtype, str) else int(src_dtype)
    n = ctypes.c_size_t(0)
    _check(load_library().flashhead_build_clusters_workspace_bytes(ctypes.byref(desc), src, ctypes.byref(n)))
    return n.value


def flashhead_build_clusters(desc: fh_desc, src_dtype, E, iters, seed, unit, centroids, cluster_tokens, workspace,
                             stream=None) -> None:
    src = DTYPES[src_dtype] if isinstance(src_dtype, str) else int(src_dtype)
    _check(load_library().flashhead_build_clusters(
        ctypes.byref(desc), src, _ptr(E), int(iters), int(seed), int(bool(unit)), _ptr(centroids),
        _ptr(cluster_tokens), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def flashhead_centroid_scores(desc: fh_desc, h, centroids, mode, temperature, seed, step, workspace,
                              keys_out=None, stream=None) -> None:
    _check(load_library().flashhead_centroid_scores(
        ctypes.byref(desc), _ptr(h), _ptr(centroids), _mode(mode), float(temperature), int(seed), int(step),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(keys_out), _stream(stream)))


def flashhead_select_probes(desc: fh_desc, p, workspace, probe_ids_out=None, stream=None) -> None:
    _check(load_library().flashhead_select_probes(
        ctypes.byref(desc), int(p), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(probe_ids_out), _stream(stream)))


def flashhead_probe_logits(desc: fh_desc, p, h, cluster_tokens, E_tiles, E_scales, mode, temperature, seed,
                           step, workspace, out: fh_outputs, stream=None) -> None:
    _check(load_library().flashhead_probe_logits(
        ctypes.byref(desc), int(p), _ptr(h), _ptr(cluster_tokens), _ptr(E_tiles), _ptr(E_scales), _mode(mode),
        float(temperature), int(seed), int(step), _ptr(workspace), workspace.numel() * workspace.element_size(),
        ctypes.byref(out), _stream(stream)))


def flashhead_select_and_probe(desc: fh_desc, p, h, cluster_tokens, E_tiles, E_scales, mode, temperature, seed,
                               step, workspace, out: fh_outputs, stream=None) -> None:
    _check(load_library().flashhead_select_and_probe(
        ctypes.byref(desc), int(p), _ptr(h), _ptr(cluster_tokens), _ptr(E_tiles), _ptr(E_scales), _mode(mode),
        float(temperature), int(seed), int(step), _ptr(workspace), workspace.numel() * workspace.element_size(),
        ctypes.byref(out), _stream(stream)))


def flashhead_forward(desc: fh_desc, h, centroids, cluster_tokens, E_tiles, E_scales, p, mode, temperature,
                      seed, step, workspace, out: fh_outputs, stream=None, workspace_bytes=None) -> None:
    wsb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(load_library().flashhead_forward(
        ctypes.byref(desc), _ptr(h), _ptr(centroids), _ptr(cluster_tokens), _ptr(E_tiles), _ptr(E_scales),
        int(p), _mode(mode), float(temperature), int(seed), int(step), _ptr(workspace), wsb,
        ctypes.byref(out), _stream(stream)))


def flashhead_dense_forward(desc: fh_desc, h, E, mode, temperature, seed, step, workspace, token, logits=None,
                            stream=None) -> None:
    _check(load_library().flashhead_dense_forward(
        ctypes.byref(desc), _ptr(h), _ptr(E), _mode(mode), float(temperature), int(seed), int(step),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(token), _ptr(logits),
        _stream(stream)))


def flashhead_mc_marginal_workspace_bytes(desc: fh_desc) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().flashhead_mc_marginal_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def flashhead_mc_marginal(desc: fh_desc, h, centroids, cluster_tokens, E_tiles, E_scales, p, temperature, seed,
                          n_sets, clip, workspace, out, stream=None) -> None:
    _check(load_library().flashhead_mc_marginal(
        ctypes.byref(desc), _ptr(h), _ptr(centroids), _ptr(cluster_tokens), _ptr(E_tiles), _ptr(E_scales), int(p),
        float(temperature), int(seed), int(n_sets), int(bool(clip)), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream)))


def flashhead_philox_words(seed, row, step, rng_stream, n0, count, words_out=None, gumbel_out=None,
                           stream=None) -> None:
    _check(load_library().flashhead_philox_words(int(seed), int(row), int(step), int(rng_stream), int(n0),
                                                 int(count), _ptr(words_out), _ptr(gumbel_out), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 4 << 20     # the static scratch of flashhead_forward_noalloc (include/flashhead.h)


def flashhead_forward_noalloc(desc: fh_desc, h, centroids, cluster_tokens, E_tiles, E_scales, p, mode, temperature,
                              seed, step, out: fh_outputs, stream=None) -> None:
    _check(load_library().flashhead_forward_noalloc(
        ctypes.byref(desc), _ptr(h), _ptr(centroids), _ptr(cluster_tokens), _ptr(E_tiles), _ptr(E_scales), int(p),
        _mode(mode), float(temperature), int(seed), int(step), ctypes.byref(out), _stream(stream)))
