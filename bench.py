#!/usr/bin/env python3
"""FlashHead head throughput on one MI355X.

Workload (default): the Gemma-3-1B head shape of the FlashHead paper's experiments
(Section 4, Table 4): B = 1, d = 1152, V = 262144 tokens in c = 16384 balanced clusters of 16,
p = 512 probes, bf16 centroids / tiles / hidden state, greedy decoding.  Inputs are the seeded
synthetic head of workloads.py with the stored balanced clustering of that head
(tests/golden/clusters_gemma.npz); centroids and tiles are built on the GPU by the library.

A step is one flashhead_forward call (centroid scores, probe selection, probe logits, token)
over one hidden state.  Calls are captured in a HIP graph that cycles through R copies of the
centroids and R distinct hidden states over the one tile array, as a decode loop does: every
call reads the centroids from HBM (R x 37.7 MB is well above the 256 MB last-level cache) and
its own probe set's tiles (R different probe sets touch ~R x 19 MB of the 604 MB tiles).
Prints one JSON line.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gemma] [--mode greedy]
       python bench.py --sweep      (clusters x probes grid at the Llama-3.2-1B head shape)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_bytes(wl, B=1):
    """Bytes a call must read at least: centroids, the kept tiles, their C2T rows, h."""
    row_of = {"f32": 4 * wl.d, "bf16": 2 * wl.d, "int4": wl.d // 2 + 2 * (wl.d // 128)}
    row = row_of[wl.e_pack]
    csz = 4 if wl.dtype == "f32" else 2
    c_bytes = wl.c * row_of[wl.c_dtype]
    tile_bytes = B * wl.p * wl.b * (row + 4)
    return c_bytes, tile_bytes, c_bytes + tile_bytes + B * wl.d * csz


def source_sha256() -> str:
    """sha256 over the library sources, the key under which counter results are stored."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "clustered_retrieval_lm_amd", "csrc", "*"))):
        with open(f, "rb") as fh_:
            h.update(fh_.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernels) -> "int | None":
    """HBM bytes per launch of `kernels` (name prefixes) from profiles/hbm_traffic_<workload>_b1.txt.

    That file holds FETCH_SIZE / WRITE_SIZE per dispatch from two rocprofv3 --pmc runs of
    this script, scaled by the factors a plain 1 GiB copy gave.  None when it is missing or
    was taken on other library sources than the ones built now.
    """
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}_b1.txt")
    if not os.path.exists(path):
        return None
    sha, found = None, {}
    for line in open(path):
        if line.startswith("source_sha256:"):
            sha = line.split(":", 1)[1].strip()
        elif line.startswith("kernel:"):
            f = line.split()
            found[f[1]] = int(f[-1].split("=")[1])
    if sha != source_sha256():
        return None
    total = 0
    for k in kernels:
        hits = [v for n, v in found.items() if n.split("<")[0] == k]
        if len(hits) != 1:
            return None
        total += hits[0]
    return total


def time_graph(torch, launch, n_calls, reps, warm_reps=2):
    """Capture n_calls launches in one graph; return seconds per call over `reps` replays."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(n_calls):          # eager warm-up on the capture stream
            launch(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_calls):
            launch(i)
    for _ in range(warm_reps):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / (reps * n_calls), g


def cpu_baseline(wl, hd, C2T, budget_s=15.0):
    """The oracle forward (fp64 NumPy) on the host cores: a bounded sample of calls."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import head as ohead
    from oracle import kmeans
    Ev = ohead.decode(hd.E, wl.dtype)
    C = kmeans.centroids_from_c2t(Ev, C2T, wl.c_dtype)
    del Ev
    tiles = ohead.pack_tiles(hd.E, wl.dtype, C2T, wl.e_pack)
    ohead.forward(hd.h, wl.dtype, C, wl.c_dtype, C2T, tiles, wl.p)        # warm-up
    n, t0 = 0, time.perf_counter()
    while True:
        ohead.forward(hd.h, wl.dtype, C, wl.c_dtype, C2T, tiles, wl.p)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or n >= 200:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    model = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": n / dt, "unit": "calls/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} greedy oracle.head.forward calls (B=1, full workload shape) in {dt:.1f} s "
                      f"on {model}"}


def run_sweep(args) -> int:
    """The clusters / probes grid of the paper's Table 7 at the Llama-3.2-1B head shape
    (d = 2048, V = 128256, bf16): c in {4008, 8016, 16032} (b = 32, 16, 8), p in {128, 256, 512},
    greedy, B = 1, timed like the main bench (graph replay over R centroid copies and R hidden
    states), with the dense head as the comparator.  Synthetic heads of the workloads recipe
    whose latent partition serves as the balanced clustering (latency does not depend on
    which balanced clustering is used).  Prints one JSON line."""
    import numpy as np
    import torch

    import workloads
    from clustered_retrieval_lm_amd import flashhead as fh
    from clustered_retrieval_lm_amd.head import DeviceHead, to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lib = fh.load_library()
    import ctypes
    d, V = 2048, 128256
    rows, dense = [], None
    for ci, c in enumerate((4008, 8016, 16032)):
        b = V // c
        R = 16
        hd = workloads.make_small(d, V, c, R, seed=500 + ci, sigma_c=0.02, sigma_n=0.01, dtype="bf16")
        C2T = np.lexsort((np.arange(V), hd.latent)).reshape(c, b).astype(np.int32)
        dev = DeviceHead.from_clusters(d, V, c, C2T, hd.E, "bf16", "bf16", "bf16", "bf16", device="cuda",
                                       keep_dense=dense is None)
        Cs = [dev.C] + [dev.C.clone() for _ in range(R - 1)]
        Hs = [to_device(hd.h[r:r + 1], "cuda") for r in range(R)]
        desc = dev.desc(1)
        for p in (128, 256, 512):
            ws = dev.workspace(1, p)
            out = dev.outputs(1, p, probes=False)
            fo = fh.make_outputs(out["token"])

            def fwd(i):
                st = lib.flashhead_forward(ctypes.byref(desc), Hs[i % R].data_ptr(), Cs[i % R].data_ptr(),
                                           dev.c2t.data_ptr(), dev.tiles.data_ptr(), None, p, 0, 1.0, 0, i,
                                           ws.data_ptr(), ws.numel(), ctypes.byref(fo),
                                           torch.cuda.current_stream().cuda_stream)
                if st != 0:
                    raise fh.FlashHeadError(st, fh.flashhead_last_error())

            t, g = time_graph(torch, fwd, 8 * R, 20, warm_reps=2)
            del g
            alg = c * d * 2 + p * b * (2 * d + 4) + 2 * d
            rows.append({"c": c, "b": b, "p": p, "us_per_call": round(t * 1e6, 2),
                         "calls_per_s": round(1.0 / t, 1), "algorithmic_bytes": alg,
                         "achieved_GBps": round(alg / t / 1e9, 1)})
            log(f"c={c} b={b} p={p}: {t * 1e6:.2f} us/call, {alg / t / 1e9:.0f} GB/s")
        if dense is None:
            dws = torch.empty(fh.flashhead_dense_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
            dtok = torch.empty(1, dtype=torch.int32, device="cuda")
            E2 = [dev.E, dev.E.clone()]

            def dense_call(i):
                st = lib.flashhead_dense_forward(ctypes.byref(desc), Hs[i % R].data_ptr(), E2[i % 2].data_ptr(), 0,
                                                 1.0, 0, i, dws.data_ptr(), dws.numel(), dtok.data_ptr(), None,
                                                 torch.cuda.current_stream().cuda_stream)
                if st != 0:
                    raise fh.FlashHeadError(st, fh.flashhead_last_error())

            t_d, g = time_graph(torch, dense_call, 20, 10, warm_reps=1)
            del g, E2
            dense = {"us_per_call": round(t_d * 1e6, 2), "bytes": V * d * 2,
                     "achieved_GBps": round(V * d * 2 / t_d / 1e9, 1)}
            log(f"dense head: {t_d * 1e6:.2f} us/call")
        del dev, Cs, Hs, hd
        torch.cuda.empty_cache()
    for r in rows:
        r["speedup_vs_dense"] = round(dense["us_per_call"] / r["us_per_call"], 2)
    print(json.dumps({"sweep": "clusters x probes (FlashHead Table 7 grid), Llama-3.2-1B head shape, bf16, "
                               "B=1, greedy, synthetic", "dense": dense, "rows": rows}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2400)
    ap.add_argument("--warmup", type=int, default=240)
    ap.add_argument("--workload", default="gemma")
    ap.add_argument("--mode", default="greedy", choices=["greedy", "sample"])
    ap.add_argument("--rotate", type=int, default=0, help="copies of the head cycled through (0: auto)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-head comparator")
    ap.add_argument("--no-mc", action="store_true", help="skip the Monte-Carlo marginal (N = 10^4 probe sets)")
    ap.add_argument("--mc-sets", type=int, default=10000, help="probe sets of the Monte-Carlo marginal")
    ap.add_argument("--sweep", action="store_true",
                    help="only the clusters x probes grid (Table 7) at the Llama-3.2-1B head shape")
    ap.add_argument("--copy-calib", action="store_true", help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: the FlashHead head is measured on a single MI355X "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", flush=True)
        return 2
    if args.sweep:
        return run_sweep(args)

    import numpy as np
    import torch

    import workloads
    from clustered_retrieval_lm_amd import flashhead as fh
    from clustered_retrieval_lm_amd.head import DeviceHead, to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    fh.load_library()
    wl = workloads.WORKLOADS[args.workload]
    cfile = {"int4_b16": "int4", "gemma_c4": "gemma"}.get(args.workload, args.workload)
    C2T = np.load(os.path.join(ROOT, "tests", "golden", f"clusters_{cfile}.npz"))["C2T"]
    log(f"workload {wl.name}: B={wl.B} d={wl.d} V={wl.V} c={wl.c} p={wl.p} {wl.dtype}/{wl.e_pack}")
    hd = workloads.make_head(wl)
    dev = DeviceHead.from_clusters(wl.d, wl.V, wl.c, C2T, hd.E, wl.dtype, wl.c_dtype, wl.e_pack, wl.dtype,
                                   device="cuda", keep_dense=not args.no_dense)
    c_bytes, tile_bytes, alg_bytes = algorithmic_bytes(wl, wl.B)
    union_frac = None
    R = args.rotate or max(2, int(np.ceil(4 * MALL_BYTES / max(alg_bytes, 1))))
    log(f"rotating {R} copies of the centroids ({R * dev.C.numel() * dev.C.element_size() / 2**30:.2f} GiB) "
        f"and {R} hidden states over one tile array ({dev.tiles.numel() / 2**30:.2f} GiB)")
    Cs = [dev.C] + [dev.C.clone() for _ in range(R - 1)]
    Ts = [dev.tiles] * R
    Ss = [dev.scales] * R
    Hs = [to_device(hd.h, "cuda")] + [to_device(workloads.make_hidden(wl, wl.B, seed=1000 + r), "cuda")
                                      for r in range(1, R)]
    B, p = wl.B, wl.p
    desc = dev.desc(B)
    ws = dev.workspace(B, p)
    out = dev.outputs(B, p, probes=False)
    fo = fh.make_outputs(out["token"])
    tau = wl.temperatures[0] if (args.mode == "sample" and wl.temperatures) else 1.0
    if B > 1:
        # at B > 1 each kept tile is read once for all rows that kept it: the bytes a call must
        # read are the union of the rows' probe sets (measured here on the R hidden states)
        ids = torch.empty(B, p, dtype=torch.int32, device="cuda")
        sizes = []
        for r in range(R):
            fh.flashhead_centroid_scores(desc, Hs[r], Cs[r], args.mode, tau, wl.sample_seed, r, ws)
            fh.flashhead_select_probes(desc, p, ws, ids)
            sizes.append(int(torch.unique(ids).numel()))
        union = float(np.mean(sizes))
        union_frac = union / (B * p)
        row_b = tile_bytes // (B * p * wl.b)
        tile_bytes = int(round(union * wl.b * row_b))
        alg_bytes = c_bytes + tile_bytes + B * wl.d * (4 if wl.dtype == "f32" else 2)
        log(f"B={B}: {union:.0f} distinct clusters kept per call on average ({B * p} probes)")
    lib = fh.load_library()
    wsb = ws.numel()
    import ctypes

    def fwd(i):
        r = i % R
        st = lib.flashhead_forward(ctypes.byref(desc), Hs[r].data_ptr(), Cs[r].data_ptr(), dev.c2t.data_ptr(),
                                   Ts[r].data_ptr(), Ss[r].data_ptr() if Ss[r] is not None else None, p,
                                   fh.MODES[args.mode], tau, wl.sample_seed, i, ws.data_ptr(), wsb,
                                   ctypes.byref(fo), torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise fh.FlashHeadError(st, fh.flashhead_last_error())

    def scores(i):
        r = i % R
        st = lib.flashhead_centroid_scores(ctypes.byref(desc), Hs[r].data_ptr(), Cs[r].data_ptr(),
                                           fh.MODES[args.mode], tau, wl.sample_seed, i, ws.data_ptr(), wsb, None,
                                           torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise fh.FlashHeadError(st, fh.flashhead_last_error())

    # ---- whole path: graph of G calls, replayed
    G = R * max(1, 120 // R)
    reps = max(1, -(-args.steps // G))
    warm = max(1, -(-args.warmup // G))
    steps = reps * G
    log(f"timing {steps} steps ({reps} replays of a {G}-call graph) after {warm * G} warm-up steps")
    torch.cuda.synchronize()
    t_call, g_fwd = time_graph(torch, fwd, G, reps, warm_reps=warm)
    calls_per_s = 1.0 / t_call
    log(f"forward: {t_call * 1e6:.2f} us/call, {calls_per_s:.0f} calls/s, "
        f"{alg_bytes / t_call / 1e9:.0f} GB/s algorithmic")
    # spread: each replay of the graph timed on its own (20 replays)
    per = []
    for _ in range(20):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        g_fwd.replay()
        a1.record()
        torch.cuda.synchronize()
        per.append(a0.elapsed_time(a1) * 1e3 / G)
    spread = {"median": round(float(np.median(per)), 3), "p10": round(float(np.percentile(per, 10)), 3),
              "p90": round(float(np.percentile(per, 90)), 3), "replays": len(per), "calls_per_replay": G}
    log(f"forward per replay: median {spread['median']:.2f} us/call (p10 {spread['p10']:.2f}, p90 {spread['p90']:.2f})")
    del g_fwd

    # warm: the same centroids and hidden state every call (the centroids stay in the
    # last-level cache) -- labelled, never the headline
    def fwd_warm(i):
        st = lib.flashhead_forward(ctypes.byref(desc), Hs[0].data_ptr(), Cs[0].data_ptr(), dev.c2t.data_ptr(),
                                   Ts[0].data_ptr(), Ss[0].data_ptr() if Ss[0] is not None else None, p,
                                   fh.MODES[args.mode], tau, wl.sample_seed, i, ws.data_ptr(), wsb,
                                   ctypes.byref(fo), torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise fh.FlashHeadError(st, fh.flashhead_last_error())

    t_warm, g_w = time_graph(torch, fwd_warm, G, max(1, reps // 2), warm_reps=1)
    del g_w
    log(f"forward, warm (no rotation): {t_warm * 1e6:.2f} us/call")

    # pure-read ceiling of this GPU: a 2 GiB streaming reduction
    big = torch.empty(1 << 29, dtype=torch.float32, device="cuda").fill_(1.0)
    for _ in range(2):
        big.sum()
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record()
    for _ in range(5):
        big.sum()
    r1.record()
    torch.cuda.synchronize()
    read_ceiling = big.numel() * 4 * 5 / (r0.elapsed_time(r1) * 1e-3) / 1e9
    ceiling_src = "torch sum over 2 GiB"
    del big
    log(f"streaming read, torch sum over 2 GiB: {read_ceiling:.0f} GB/s")

    # ---- the two halves of a call, each timed alone the same way: stage 1 (k_b1_scores) and
    # selection + stage 2 (k_b1_stage2 + the one-block token decode), the latter over R
    # workspaces that hold the stage-1 keys of the R hidden states
    t_sc, g_sc = time_graph(torch, scores, G, reps, warm_reps=1)
    sc_bytes = c_bytes + B * wl.d * 2 + B * wl.c * 4
    log(f"centroid scores: {t_sc * 1e6:.2f} us/launch, {sc_bytes / t_sc / 1e9:.0f} GB/s")
    del g_sc
    wss = [torch.empty_like(ws) for _ in range(R)]
    for r in range(R):
        st = lib.flashhead_centroid_scores(ctypes.byref(desc), Hs[r].data_ptr(), Cs[r].data_ptr(),
                                           fh.MODES[args.mode], tau, wl.sample_seed, r, wss[r].data_ptr(), wsb,
                                           None, torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise fh.FlashHeadError(st, fh.flashhead_last_error())
    torch.cuda.synchronize()

    def stage2(i):
        r = i % R
        st = lib.flashhead_select_and_probe(ctypes.byref(desc), p, Hs[r].data_ptr(), dev.c2t.data_ptr(),
                                            Ts[r].data_ptr(), Ss[r].data_ptr() if Ss[r] is not None else None,
                                            fh.MODES[args.mode], tau, wl.sample_seed, r, wss[r].data_ptr(), wsb,
                                            ctypes.byref(fo), torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise fh.FlashHeadError(st, fh.flashhead_last_error())

    t_s2, g_s2 = time_graph(torch, stage2, G, reps, warm_reps=1)
    s2_bytes = tile_bytes + B * wl.c * 4 + B * wl.d * 2
    log(f"selection + stage 2: {t_s2 * 1e6:.2f} us/call, {s2_bytes / t_s2 / 1e9:.0f} GB/s")
    del g_s2, wss

    dense = None
    if not args.no_dense:
        dws = torch.empty(fh.flashhead_dense_workspace_bytes(dev.desc(B, e_dtype=wl.dtype)), dtype=torch.uint8,
                          device="cuda")
        dtok = torch.empty(B, dtype=torch.int32, device="cuda")
        ddesc = dev.desc(B, e_dtype=wl.dtype)
        E2 = [dev.E, dev.E.clone()]

        def dense_call(i):
            st = lib.flashhead_dense_forward(ctypes.byref(ddesc), Hs[i % R].data_ptr(), E2[i % 2].data_ptr(),
                                             fh.MODES[args.mode], tau, wl.sample_seed, i, dws.data_ptr(),
                                             dws.numel(), dtok.data_ptr(), None,
                                             torch.cuda.current_stream().cuda_stream)
            if st != 0:
                raise fh.FlashHeadError(st, fh.flashhead_last_error())

        t_d, g_d = time_graph(torch, dense_call, 20, 10, warm_reps=1)
        dense_bytes = wl.V * wl.d * (2 if wl.dtype == "bf16" else 4)
        # secondary comparator: torch's linear + argmax on the same E (its library GEMV/GEMM)
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        Et = [x.view(tdt).view(wl.V, wl.d) for x in E2]
        Ht = [x.view(tdt).view(B, wl.d) for x in Hs]

        def torch_call(i):
            torch.argmax(torch.nn.functional.linear(Ht[i % R], Et[i % 2]), dim=-1)

        t_t, g_t = time_graph(torch, torch_call, 20, 10, warm_reps=1)
        del g_t, Et, Ht
        dense = {"calls_per_s": round(1.0 / t_d, 1), "us_per_call": round(t_d * 1e6, 2),
                 "achieved_GBps": round(dense_bytes / t_d / 1e9, 1), "bytes": dense_bytes,
                 "speedup": round(t_d / t_call, 2), "byte_ratio": round(dense_bytes / alg_bytes, 2),
                 "torch_linear_argmax_us": round(t_t * 1e6, 2)}
        log(f"torch linear + argmax on the same E: {t_t * 1e6:.1f} us/call")
        if dense_bytes / t_d / 1e9 > read_ceiling:         # the dense GEMV streams E at a higher rate
            read_ceiling = dense_bytes / t_d / 1e9
            ceiling_src = f"flashhead_dense_forward streaming {dense_bytes / 1e6:.0f} MB"
        log(f"dense head: {t_d * 1e6:.1f} us/call, {dense_bytes / t_d / 1e9:.0f} GB/s; "
            f"FlashHead speedup {t_d / t_call:.2f}x (byte ratio {dense_bytes / alg_bytes:.2f}x)")
        del g_d, E2

    mc = None
    if not args.no_mc:
        # Appendix D.1's estimator: N probe sets per hidden state, the whole-vocabulary estimate
        mws = torch.empty(fh.flashhead_mc_marginal_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        mout = torch.empty(B, wl.V, dtype=torch.float64, device="cuda")
        n_mc = args.mc_sets

        def mc_call(i):
            fh.flashhead_mc_marginal(desc, Hs[i % R], Cs[i % R], dev.c2t, Ts[i % R], Ss[i % R], p, 1.0,
                                     wl.sample_seed, n_mc, True, mws, mout)

        mc_call(0)
        torch.cuda.synchronize()
        reps_mc = 5
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps_mc):
            mc_call(i)
        e1.record()
        torch.cuda.synchronize()
        t_mc = e0.elapsed_time(e1) / 1e3 / reps_mc
        mc = {"n_sets": n_mc, "p": p, "tau": 1.0, "ms_per_call": round(t_mc * 1e3, 3),
              "sets_per_s": round(B * n_mc / t_mc, 0), "us_per_set": round(t_mc * 1e6 / (B * n_mc), 4)}
        log(f"Monte-Carlo marginal: {n_mc} probe sets in {t_mc * 1e3:.2f} ms "
            f"({B * n_mc / t_mc:.3g} sets/s)")
        del mws, mout

    if args.copy_calib:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b_ = torch.empty_like(a)
        for _ in range(3):
            b_.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies")

    cpu = None
    if not args.no_cpu:
        log("oracle baseline on the host cores ...")
        cpu = cpu_baseline(wl, hd, C2T)
        log(f"oracle: {cpu['value']:.2f} calls/s on {cpu['cores']} threads")

    if B == 1:
        units = {
            "k_b1_scores (centroid scores)": (sc_bytes, t_sc, ["fh::k_b1_scores"]),
            "k_b1_stage2 + k_finalize_parts (selection, probe logits, token)":
                (s2_bytes, t_s2, ["fh::k_b1_stage2", "fh::k_finalize_parts"]),
        }
    else:
        units = {
            "k_mfma / k_scores_gemv (centroid scores)": (sc_bytes, t_sc, ["fh::k_mfma", "fh::k_scores_gemv"]),
            "k_select + k_tiles_mask + k_finalize (selection, probe logits, tokens)":
                (s2_bytes, t_s2, ["fh::k_select", "fh::k_tiles_mask", "fh::k_finalize"]),
        }
    dom = max(units, key=lambda k: units[k][1])
    dom_bytes, dom_t, dom_kernels = units[dom]
    dom_gbs = dom_bytes / dom_t / 1e9
    traffic = measured_traffic(args.workload, dom_kernels) if args.mode == "greedy" else None
    res = {
        "metric": "head calls/s + achieved HBM GB/s vs dense LM head, B=1 Gemma-3-1B shape",
        "value": round(calls_per_s, 1),
        "unit": "calls/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm * G,
        "ms_per_step": round(t_call * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name} head (B={B}, d={wl.d}, V={wl.V}, c={wl.c}, b={wl.b}, p={p}, "
                               f"{wl.c_dtype} C, {wl.dtype} h, {wl.e_pack} tiles, {args.mode})",
                   "mode": args.mode, "rotated_copies": R},
        "achieved_GBps": round(alg_bytes / t_call / 1e9, 1),
        "algorithmic_bytes": alg_bytes,
        "us_per_call_spread": spread,
        "warm_us_per_call": round(t_warm * 1e6, 3),
        "read_ceiling": {"GBps": round(read_ceiling, 1), "source": ceiling_src,
                         "frac": round(alg_bytes / t_call / 1e9 / read_ceiling, 4)},
        "kept_union_fraction": None if union_frac is None else round(union_frac, 4),
        # the batched centroid GEMM on MFMA (B > 1, bf16): its arithmetic rate against the dense
        # bf16 MFMA peak (it is bound by the centroid bytes: B flop per byte read)
        "stage1_mfma": None if B == 1 else {
            "tflops": round(2.0 * B * wl.c * wl.d / t_sc / 1e12, 2), "peak_tflops": 2500.0,
            "frac": round(2.0 * B * wl.c * wl.d / t_sc / 1e12 / 2500.0, 5)},
        "roofline": {"bound": "hbm", "kernel": dom,
                     "achieved": round(dom_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": dom_bytes, "us_per_launch": round(dom_t * 1e6, 3)},
        "kernels": {k: {"bytes_per_launch": b_, "us_per_launch": round(t_ * 1e6, 3),
                        "GBps": round(b_ / t_ / 1e9, 1)} for k, (b_, t_, _) in units.items()},
        "dense": dense,
        "mc_marginal": mc,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
