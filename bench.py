#!/usr/bin/env python3
"""Benchmark: fused decode-GEMV on compressed BF16 weights, batch 1, one MI355X.

One step = the batch-1 GEMVs of one Qwen3-4B-shaped decoder layer (q, k, v,
o, gate, up, down; seeded synthetic weights, x ~ N(0, 1)), run in the order a
decode step needs them.  Inputs are resident in HBM before timing starts.
To measure HBM rather than the 256 MB Infinity Cache, steps cycle through
several device copies of the layer (>= 1 GB in total).  Each copy's step is
captured once as a HIP graph and replayed.

Prints ONE JSON line.  `value` is compressed GB/s (blob + x + y bytes per
step / step time); the uncompressed-equivalent rate, % of HBM peak, the same
GEMV reading plain BF16, the roofline figure of the dominant kernel and the
CPU oracle's rate on a bounded sample are reported beside it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, help="workload id (1..5); 2 = Qwen3-4B-shaped layer")
    ap.add_argument("--copies", type=int, default=0, help="device copies cycled (0 = enough for >= 1 GB)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--roofline-reps", type=int, default=200)
    ap.add_argument("--skip-bf16", action="store_true")
    ap.add_argument("--tile-rows", type=int, default=0, help="encoder tile rows (0 = library default)")
    ap.add_argument("--max-code-len", type=int, default=0, help="encoder code length limit (0 = library default)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(row-sharding across GPUs is described in DESIGN.md but not built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import decode_gemv_byte_amd as nwc
    import workloads

    torch.cuda.set_device(0)
    wl = workloads.WORKLOADS[args.workload]
    if wl.layers != 1 and args.workload != 3:
        pass
    layer_ids = [0]
    mats = list(wl.matrices)
    order = [m for g in wl.groups for m in g] if wl.groups else [m.name for m in mats]

    # ---------------------------------------------------------------- setup
    t0 = time.time()
    host = {}
    for m in mats:
        w = workloads.weights(wl.cid, m.name, layer=0)
        params = {k: v for k, v in (("tile_rows", args.tile_rows), ("max_code_len", args.max_code_len)) if v}
        blob = nwc.nwc_encode(w, params or None)
        host[m.name] = (w, blob, nwc.nwc_inspect(blob))
    enc_s = time.time() - t0
    bytes_c = sum(host[n][1].size + 2 * host[n][2].cols + 2 * host[n][2].rows for n in order)
    bytes_u = sum(2 * host[n][2].rows * host[n][2].cols + 2 * host[n][2].cols + 2 * host[n][2].rows
                  for n in order)
    blob_bytes = sum(host[n][1].size for n in order)
    copies = args.copies or max(1, int(np.ceil(1.0e9 / blob_bytes)))

    dev = torch.device("cuda", 0)
    blobs = [{n: torch.from_numpy(host[n][1]).to(dev) for n in order} for _ in range(copies)]
    xs = {n: torch.from_numpy(workloads.activations(wl.cid, n)[0]).to(dev) for n in order}
    ys = {n: torch.empty(host[n][2].rows, dtype=torch.bfloat16, device=dev) for n in order}
    infos = {n: host[n][2] for n in order}
    stream = torch.cuda.Stream()

    def zeroed_ws(names):
        # the fused path's workspace: zero-filled once, left zero by every call
        return torch.zeros(nwc.gemv_batched_workspace_size([infos[n] for n in names]), dtype=torch.uint8,
                           device=dev)

    # one launch per dependency group (GEMVs that read the same activations);
    # launches are stream-ordered, so each group's workspace serves every copy
    groups = [list(g) for g in wl.groups] if wl.groups else [[n] for n in order]
    gws = [zeroed_ws(g) for g in groups]
    batches = [[nwc.GemvBatch([infos[n] for n in g], [blobs[c][n] for n in g], [xs[n] for n in g],
                              [ys[n] for n in g], gws[k]) for k, g in enumerate(groups)] for c in range(copies)]

    def step(c):
        for bt in batches[c]:
            nwc.nwc_gemv_batched(bt, stream=stream)

    # correctness guard: one eager step, compared with an FP64 reference of
    # the BF16 values computed by torch on the host (not timed)
    with torch.cuda.stream(stream):
        step(0)
    torch.cuda.synchronize()
    for n in order:
        w = host[n][0]
        wf = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).double()
        xf = xs[n].cpu().view(torch.bfloat16).double()
        ref = (wf @ xf).numpy()
        a = (wf.abs() @ xf.abs()).numpy()
        got = ys[n].cpu().double().numpy()
        ok = np.all(np.abs(got - ref) <= 2.0 ** -10 * a + 2.0 ** -8 * np.abs(ref))
        if not ok:
            print("bench: GEMV %s outside tolerance" % n, file=sys.stderr)
            sys.exit(1)

    graphs = None
    if not args.no_graph:
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(c)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(k, start):
        for i in range(k):
            c = (start + i) % copies
            if graphs is not None:
                with torch.cuda.stream(stream):
                    graphs[c].replay()
            else:
                with torch.cuda.stream(stream):
                    step(c)

    # --------------------------------------------------------------- timed
    run(args.warmup, 0)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    ev0.record(stream)
    run(args.steps, args.warmup)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_start
    ms_gpu = ev0.elapsed_time(ev1)
    ms_per_step = ms_gpu / args.steps
    value = bytes_c * args.steps / (ms_gpu * 1e-3) / 1e9
    value_u = bytes_u * args.steps / (ms_gpu * 1e-3) / 1e9

    # ------------------------------------------- dominant kernel, roofline
    # the dominant kernel is the launch that moves the most bytes; its average
    # duration is measured with events on the launch stream over back-to-back
    # launches cycling the device copies
    gbytes = [sum(host[n][1].size + 2 * infos[n].cols + 2 * infos[n].rows for n in g) for g in groups]
    gi = int(np.argmax(gbytes))
    dom_bytes = gbytes[gi]
    reps = args.roofline_reps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for i in range(10):
            nwc.nwc_gemv_batched(batches[i % copies][gi], stream=stream)
        e0.record(stream)
        for i in range(reps):
            nwc.nwc_gemv_batched(batches[i % copies][gi], stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    dom_us = e0.elapsed_time(e1) * 1e3 / reps
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9

    # all seven GEMVs in one launch: they read independent activations here
    iws = zeroed_ws(order)
    indep = [nwc.GemvBatch([infos[n] for n in order], [blobs[c][n] for n in order], [xs[n] for n in order],
                           [ys[n] for n in order], iws) for c in range(copies)]
    with torch.cuda.stream(stream):
        for i in range(10):
            nwc.nwc_gemv_batched(indep[i % copies], stream=stream)
        e0.record(stream)
        for i in range(reps):
            nwc.nwc_gemv_batched(indep[i % copies], stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    indep_us = e0.elapsed_time(e1) * 1e3 / reps

    # ------------------------------------------------ plain BF16 comparator
    bf16 = None
    if not args.skip_bf16:
        wdev = {n: [torch.from_numpy(host[n][0].view(np.int16)).to(dev) for _ in range(copies)] for n in order}
        wsb = {n: torch.empty(nwc.nwc_bf16_workspace_size(infos[n].rows, infos[n].cols), dtype=torch.uint8,
                              device=dev) for n in order}
        yb = {n: torch.empty(infos[n].rows, dtype=torch.bfloat16, device=dev) for n in order}

        def step_bf16(c):
            for n in order:
                nwc.nwc_gemv_bf16(wdev[n][c], xs[n], yb[n], wsb[n], stream=stream)

        gb = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step_bf16(c)
            gb.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            with torch.cuda.stream(stream):
                gb[i % copies].replay()
        torch.cuda.synchronize()
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for i in range(args.steps):
            with torch.cuda.stream(stream):
                gb[i % copies].replay()
        b1.record(stream)
        torch.cuda.synchronize()
        ms_b = b0.elapsed_time(b1) / args.steps
        bf16 = dict(ms_per_step=round(ms_b, 5), GBps=round(bytes_u / (ms_b * 1e-3) / 1e9, 1),
                    speedup_fused_vs_bf16=round(ms_b / ms_per_step, 3))

        # the vendor library's BF16 GEMV (torch.mv), same matrices, same launch
        # order, also graph-captured: an outside reference
        wt = {n: [w.view(torch.bfloat16) for w in wdev[n]] for n in order}
        xt = {n: xs[n].view(torch.bfloat16) for n in order}
        yt = {n: torch.empty(infos[n].rows, dtype=torch.bfloat16, device=dev) for n in order}

        def step_torch(c):
            for n in order:
                torch.mv(wt[n][c], xt[n], out=yt[n])

        with torch.cuda.stream(stream):
            step_torch(0)
        torch.cuda.synchronize()
        gt = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step_torch(c)
            gt.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            with torch.cuda.stream(stream):
                gt[i % copies].replay()
        torch.cuda.synchronize()
        b0.record(stream)
        for i in range(args.steps):
            with torch.cuda.stream(stream):
                gt[i % copies].replay()
        b1.record(stream)
        torch.cuda.synchronize()
        ms_t = b0.elapsed_time(b1) / args.steps
        bf16["torch_mv"] = dict(ms_per_step=round(ms_t, 5), GBps=round(bytes_u / (ms_t * 1e-3) / 1e9, 1),
                                    speedup_fused_vs_torch=round(ms_t / ms_per_step, 3))
        del wdev, wt

    # ------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(host, order, args.cpu_seconds)

    out = {
        "metric": "fused decode-GEMV GB/s (compressed + uncompressed-equiv), % HBM peak, batch 1",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "matrices": {n: [infos[n].rows, infos[n].cols] for n in order},
                   "batch": 1, "launch_order": [list(g) for g in wl.groups], "device_copies": copies,
                   "hip_graph": graphs is not None, "output": "bf16"},
        "compressed_GBps": round(value, 1),
        "uncompressed_equiv_GBps": round(value_u, 1),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "bytes_per_step": {"compressed": int(bytes_c), "uncompressed": int(bytes_u)},
        "bf16_gemv": bf16,
        "single_launch_7_gemvs": {"us": round(indep_us, 3),
                                  "compressed_GBps": round(bytes_c / (indep_us * 1e-6) / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "k_gemv via nwc_gemv_batched (%s)" % "+".join(groups[gi]),
                     "bytes_per_launch": int(dom_bytes), "avg_launch_us": round(dom_us, 3)},
        "cpu_baseline": cpu,
        "wall_s": round(t_wall, 3),
        "encode_s": round(enc_s, 2),
    }
    print(json.dumps(out))


def cpu_baseline(host, order, seconds):
    """The oracle (single-threaded C: bit-serial decode + FP64 GEMV) on a
    bounded sample: row blocks of each matrix, round robin, until `seconds`
    of CPU work; rate in compressed bytes per second of the sampled rows."""
    import oracle
    import workloads  # noqa: F401

    t_total = 0.0
    bytes_done = 0.0
    rows_done = 0
    i = 0
    blocks = {}
    while t_total < seconds and i < 1000:
        n = order[i % len(order)]
        w = host[n][0]
        nb = 256
        r0 = (i // len(order)) * nb % w.shape[0]
        sub = np.ascontiguousarray(w[r0:r0 + nb])
        key = (n, r0)
        if key not in blocks:
            blocks[key] = oracle.encode(sub, 8, 512, 64, 12)
        blob = blocks[key]
        x = np.zeros(sub.shape[1], np.uint16) + np.uint16(0x3F80)
        t = time.perf_counter()
        wd = oracle.decode(blob)
        oracle.gemv(wd, x)
        t_total += time.perf_counter() - t
        bytes_done += blob.size + 2 * sub.shape[1] + 2 * sub.shape[0]
        rows_done += sub.shape[0]
        i += 1
    return {"value": round(bytes_done / t_total / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d row blocks of 256 rows from the layer's matrices, oracle decode + FP64 GEMV, "
                      "%.1f s of single-thread CPU time" % (i, t_total)}


if __name__ == "__main__":
    main()
