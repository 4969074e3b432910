"""Build libflashhead.so for gfx950 with hipcc (in-tree, no JIT cache).

usage: python -m clustered_retrieval_lm_amd.build [--verbose]
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libflashhead.so")
# (source, object name, extra flags): fh_b1.hip is compiled once per row format so that the
# three formats' B = 1 kernels build in parallel
SOURCES = [
    ("fh_kernels.hip", "fh_kernels", []),
    ("fh_b1.hip", "fh_b1_f32", ["-DFH_B1_RF=0"]),
    ("fh_b1.hip", "fh_b1_bf16", ["-DFH_B1_RF=1"]),
    ("fh_b1.hip", "fh_b1_int4", ["-DFH_B1_RF=2"]),
    ("fh_cluster.hip", "fh_cluster", []),
    ("fh_mc.hip", "fh_mc", []),
    ("fh_util.hip", "fh_util", []),
    ("fh_api.hip", "fh_api", []),
]
HEADERS = ["fh_device.h", "fh_internal.h", "fh_rows.h", "fh_select.h"]
ARCH = os.environ.get("FLASHHEAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def _run(cmd: list) -> subprocess.Popen:
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _messages(out: str) -> list:
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless.
    noise = "is not a recognized feature for this target"
    return [ln for ln in out.splitlines() if noise not in ln]


def build(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel) and link LIB; returns its path.  Always recompiles."""
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    objs, procs = [], []
    for s, name, extra in SOURCES:
        obj = os.path.join(objdir, name + ".o")
        cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, s), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        objs.append(obj)
        procs.append((name, _run(cmd)))
    failed, msgs = [], []
    for s, pr in procs:
        out, _ = pr.communicate()
        m = _messages(out)
        if pr.returncode != 0:
            failed.append(s)
        msgs += m
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(failed)}:\n" + "\n".join(msgs))
    tmp = LIB + ".tmp"
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    res = subprocess.run(link, capture_output=True, text=True)
    msgs += _messages(res.stdout + res.stderr)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
