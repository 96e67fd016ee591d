#!/usr/bin/env python3
"""Benchmark: fused decode-GEMV on compressed BF16 weights, one MI355X.

Default workload (3): one batch-1 decode step of a Llama-3.1-8B-shaped
model, the largest single-GPU batch-1 workload: 32 layers of q, k, v, o,
gate, up, down (seeded synthetic weights with 0.1% outliers, x ~ N(0, 1)),
launched in the order a decode step needs them, GEMVs that read the same
activations sharing a launch (128 launches, one graph).  Other workloads:
  1  one 1024x1024 matrix, batch 1
  2  one Qwen3-4B-shaped decoder layer, batch 1
  4  skinny decode-GEMM, 4096x14336 and 14336x4096, --batch 2..32 (more: decode + hipBLASLt)
  5  LM head 128256x4096, --batch 1 or 8

Inputs are resident in HBM before timing starts.  To measure HBM rather than
the 256 MB Infinity Cache, steps cycle through device copies of the
compressed weights (>= 1 GB in total).  Each copy's step is captured once as
a HIP graph and replayed.

Prints ONE JSON line.  `value` is compressed GB/s (blob + x + y bytes per step
/ step time); the uncompressed-equivalent rate, % of HBM peak, the same GEMVs
reading plain BF16 (our kernel and torch's), the HBM read rate a plain
streaming kernel reaches on this GPU (read probe), the roofline figure of the
dominant kernel and the CPU oracle's rate on a bounded sample (one thread and
all host cores) sit beside it.

--roofline-only runs just the dominant launch (warm-up + timed repetitions),
so that a profiler's per-kernel statistics cover exactly that launch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_TFLOPS = 2500.0   # dense BF16 matrix-core peak
STREAM_BYTES = 1.0e9          # device copies cycled per pass, well above the Infinity Cache
CHECK_ROWS = 256              # rows per matrix checked against an FP64 product
PROBE_BYTES = 4 << 30         # read-probe buffer, 16x the Infinity Cache
DEFAULT_PAIR_FIT = 1024       # the library's default 6-bit cap of common exponents (nwc_params.pair_fit)
KERNEL_SRC = os.path.join(ROOT, "decode_gemv_byte_amd", "csrc", "kernels.hip")
SETTLE_MS = 50.0              # GPU time of work run before each timed loop (clocks settle)


def note(msg):
    """A progress line on stderr (the JSON result is the one stdout line)."""
    print("[bench] " + msg, file=sys.stderr, flush=True)


def settle(torch, stream, launch, ms=SETTLE_MS):
    """Keep the GPU busy with launch(i) (one launch or one graph replay on
    `stream`) for at least `ms` of GPU time, so that a timed loop starts at
    settled clocks: on an MI355X that was idle, the first few milliseconds
    of load run up to ~15% slower (gate+up of the Llama step: 42.9 us per
    launch over its first ~9 ms of launches, 36.7-36.9 us afterwards, eager
    or graph-replayed alike).  Returns the launches run."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n, done, batch = 0, 0.0, 4
    while done < ms:
        with torch.cuda.stream(stream):
            e0.record(stream)
            for i in range(batch):
                launch(n + i)
            e1.record(stream)
        torch.cuda.synchronize()
        n += batch
        done += e0.elapsed_time(e1)
        batch = min(2 * batch, 1 << 14)
    return n


def traffic_file(workload_name, group):
    return os.path.join(ROOT, "profiles", "k_gemv_%s_%s_traffic.txt" % (workload_name, "_".join(group)))


def host_threads():
    """Host threads this process may use: the cores it is pinned to, capped
    by OMP_NUM_THREADS when that is set (a shared GPU machine sets it to its
    CPU share)."""
    n = len(os.sched_getaffinity(0))
    try:
        n = min(n, int(os.environ["OMP_NUM_THREADS"]))
    except (KeyError, ValueError):
        pass
    return max(1, n)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=3, help="1..5; 3 = Llama-3.1-8B-shaped step (default)")
    ap.add_argument("--batch", type=int, default=0, help="batch size (0 = the workload's first)")
    ap.add_argument("--copies", type=int, default=0, help="device copies cycled (0 = enough for >= 1 GB)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time of each oracle baseline leg (one thread; all host cores)")
    ap.add_argument("--roofline-reps", type=int, default=200)
    ap.add_argument("--roofline-only", action="store_true", help="time only the dominant launch")
    ap.add_argument("--skip-bf16", action="store_true", help="skip the plain-BF16 comparators")
    ap.add_argument("--force-prefill", action="store_true",
                    help="batches above 1 through decode + hipBLASLt even where the skinny GEMM takes them")
    ap.add_argument("--tile-rows", type=int, default=0, help="encoder tile rows (0 = library default)")
    ap.add_argument("--max-code-len", type=int, default=0, help="encoder code length limit (0 = library default)")
    ap.add_argument("--pair-fit", type=int, default=0, metavar="K",
                    help="encoder: exponents held by at least 1/K of the weights get codes of at most 6 bits")
    ap.add_argument("--code-family", choices=("huffman", "unary"), default="huffman",
                    help="encoder code family: length-limited Huffman (default) or the ranked unary code with an "
                         "escape (with --max-code-len 0 it takes a 12-bit limit)")
    ap.add_argument("--geometry", choices=("default", "tuned"), default="default",
                    help="tuned: time every candidate tile geometry per launch group on this GPU first "
                         "(decode_gemv_byte_amd.tune) and encode each group with the fastest")
    ap.add_argument("--model-step", type=int, default=0, metavar="LAYERS",
                    help="only time a whole decode step (tokens/s) through a Qwen3-4B-shaped stack of LAYERS "
                         "layers on synthetic weights, compressed vs dense BF16")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB, 5 times (scales HBM byte counters)")
    ap.add_argument("--probe-only", action="store_true", help="only run the HBM read probe")
    return ap.parse_args()


def model_step(args):
    """One generated token through a Qwen3-4B-shaped decoder stack (hidden 2560,
    32 query / 8 key-value heads of 128, MLP 9728): per layer RMSNorm, q/k/v in
    one batched fused launch, attention over a fixed synthetic BF16 KV cache
    of 512 positions (torch products), o, residual, RMSNorm, gate/up in
    one launch, SiLU * up, down, residual.  The projections run compressed
    (nwc_gemv_batched / nwc_gemv) or, for comparison, as torch.mv on the
    same BF16 weights; everything else is the same torch code.  Weights are
    the qwen3_4b_layer matrices, one device copy per layer (so every layer streams
    from HBM); the KV cache is random and not appended to.  The step is
    captured as one HIP graph.  Reports tokens/s (= steps/s, batch 1)."""
    import torch
    import torch.nn.functional as F

    import decode_gemv_byte_amd as nwc
    import workloads

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    L, CTX, H, HQ, HKV, D = args.model_step, 512, 2560, 32, 8, 128
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    w = {n: workloads.weights(2, n) for n in names}
    enc = {n: None for n in names}
    tuned = None
    if getattr(args, "geometry", "default") == "tuned":   # per launch group, as the main bench does
        from decode_gemv_byte_amd import tune
        tuned = {}
        for grp in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
            r = tune.tune_geometry([w[n] for n in grp])
            tuned["+".join(grp)] = r.params()
            for n in grp:
                enc[n] = r.params()
    blob = {n: nwc.nwc_encode(w[n], enc[n]) for n in names}
    info = {n: nwc.nwc_inspect(blob[n]) for n in names}
    lay = []
    for l in range(L):
        d = {n: torch.from_numpy(blob[n]).to(dev) for n in names}
        d.update({"w_" + n: torch.from_numpy(w[n].view(np.int16)).to(dev).view(torch.bfloat16) for n in names})
        lay.append(d)
    g = torch.Generator(device="cpu").manual_seed(5)
    # KV cache in BF16 as a server keeps it: K^T [kv head, dim, position] with
    # the 1/sqrt(head dim) score scale folded in, V [kv head, position, dim]
    kt = [(torch.randn(HKV, D, CTX, generator=g) / math.sqrt(D)).to(torch.bfloat16).to(dev).contiguous()
          for _ in range(L)]
    vv = [torch.randn(HKV, CTX, D, generator=g).to(torch.bfloat16).to(dev).contiguous() for _ in range(L)]
    x0 = torch.randn(H, generator=g).to(dev).to(torch.bfloat16)
    bufs = {n: torch.empty(info[n].rows, dtype=torch.bfloat16, device=dev) for n in names}
    ws_qkv = torch.zeros(nwc.gemv_batched_workspace_size([info[n] for n in ("q", "k", "v")]), dtype=torch.uint8, device=dev)
    ws_gu = torch.zeros(nwc.gemv_batched_workspace_size([info["gate"], info["up"]]), dtype=torch.uint8, device=dev)
    ws_o = torch.zeros(nwc.nwc_workspace_size(info["o"], 1), dtype=torch.uint8, device=dev)
    ws_d = torch.zeros(nwc.nwc_workspace_size(info["down"], 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    act = torch.empty(9728, dtype=torch.bfloat16, device=dev)
    x = x0.clone()
    keep = []   # marshalled launch arguments referenced by the captured graph

    def attention(l):
        # one query token against the cache, 4 query heads per KV head; BF16
        # operands (all contiguous), FP32 accumulation inside the products
        q = bufs["q"].view(HKV, HQ // HKV, D)
        p_ = torch.softmax(torch.matmul(q, kt[l]), dim=-1)               # [8, 4, CTX]
        return torch.matmul(p_, vv[l]).view(-1)                          # [4096]

    def step(dense):
        for l in range(L):
            d = lay[l]
            h = F.rms_norm(x, (H,), eps=1e-6)
            if dense:
                for n in ("q", "k", "v"):
                    torch.mv(d["w_" + n], h, out=bufs[n])
            else:
                b = nwc.GemvBatch([info[n] for n in ("q", "k", "v")], [d[n] for n in ("q", "k", "v")], [h, h, h],
                                  [bufs["q"], bufs["k"], bufs["v"]], ws_qkv)
                keep.append(b)
                nwc.nwc_gemv_batched(b, stream=stream)
            att = attention(l)
            if dense:
                torch.mv(d["w_o"], att, out=bufs["o"])
            else:
                keep.append(att)
                nwc.nwc_gemv(info["o"], d["o"], att, bufs["o"], ws_o, stream=stream)
            x.add_(bufs["o"])
            h = F.rms_norm(x, (H,), eps=1e-6)
            if dense:
                torch.mv(d["w_gate"], h, out=bufs["gate"])
                torch.mv(d["w_up"], h, out=bufs["up"])
            else:
                b = nwc.GemvBatch([info["gate"], info["up"]], [d["gate"], d["up"]], [h, h],
                                  [bufs["gate"], bufs["up"]], ws_gu)
                keep.append(b)
                nwc.nwc_gemv_batched(b, stream=stream)
            torch.mul(F.silu(bufs["gate"]), bufs["up"], out=act)
            if dense:
                torch.mv(d["w_down"], act, out=bufs["down"])
            else:
                nwc.nwc_gemv(info["down"], d["down"], act, bufs["down"], ws_d, stream=stream)
            x.add_(bufs["down"])

    res = {}
    outs = {}
    replays_match = {}
    for dense in (False, True):
        with torch.cuda.stream(stream):
            x.copy_(x0)
            step(dense)   # eager once (also fixes the workspaces' state)
        torch.cuda.synchronize()
        eager = x.float().cpu().clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step(dense)
        with torch.cuda.stream(stream):
            x.copy_(x0)
            graph.replay()
        torch.cuda.synchronize()
        outs[dense] = x.float().cpu().clone()
        settle(torch, stream, lambda i: graph.replay())
        for i in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for i in range(args.steps):
                graph.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        res[dense] = e0.elapsed_time(e1) / args.steps
        # a replay after many others still gives the eager step's bits
        with torch.cuda.stream(stream):
            x.copy_(x0)
            graph.replay()
        torch.cuda.synchronize()
        replays_match[dense] = bool(torch.equal(eager, outs[dense]) and torch.equal(eager, x.float().cpu()))
        del graph
    # the two stacks run the same arithmetic up to rounding of the products:
    # after L layers the hidden states still agree closely
    rel = float((outs[False] - outs[True]).norm() / outs[True].norm())
    comp = sum(b.size for b in blob.values()) * L
    dense_bytes = sum(2 * w[n].size for n in names) * L
    line = {
        "metric": "decode step tokens/s, batch 1 (Qwen3-4B-shaped stack, synthetic weights)",
        "value": round(1e3 / res[False], 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(res[False], 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qwen3_4b_stack", "layers": L, "context": CTX, "batch": 1, "hip_graph": True,
                   "encoder": {"tuned": tuned} if tuned else "default",
                   "weights": "qwen3_4b_layer matrices, one device copy per layer"},
        "dense_bf16_torch_mv": {"tokens_per_s": round(1e3 / res[True], 2), "ms_per_step": round(res[True], 4)},
        "speedup_vs_dense": round(res[True] / res[False], 3),
        "weight_bytes": {"compressed": int(comp), "bf16": int(dense_bytes)},
        "final_hidden_rel_diff_vs_dense": round(rel, 5),
        "graph_replays_match_eager": {"compressed": replays_match[False], "dense": replays_match[True]}}
    print(json.dumps(line))
    return line


def copy_calibration(mib):
    """A plain copy of known size: what FETCH_SIZE and WRITE_SIZE read for it
    gives the factors that turn those counters into HBM bytes."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    for i in range(5):
        dst[i % 2].copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "reps": 5}))


def traffic_from_profile(path):
    """Measured HBM bytes per dominant launch (FETCH_SIZE + WRITE_SIZE, each
    scaled by a copy kernel of known size), if the kernels have not changed
    since the counters were taken; else None."""
    try:
        text = open(path).read()
    except OSError:
        return None
    fields = dict(l.split(":", 1) for l in text.splitlines() if ":" in l and not l.startswith("#"))
    digest = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if fields.get("kernels.hip sha256", "").strip() != digest:
        return None
    try:
        return int(float(fields["hbm bytes per launch"]))
    except (KeyError, ValueError):
        return None


def read_probe(torch, nwc, stream, reps=20):
    """HBM read rate of a plain streaming kernel (nwc_read_probe) over a 4 GiB
    buffer, 16x the Infinity Cache: the fastest of two layouts (grid-stride;
    one contiguous range per workgroup) at four launch sizes, each averaged
    over `reps` back-to-back launches timed with HIP events on the probe's
    stream, after the clocks have settled."""
    buf = torch.ones(PROBE_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    best = None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    settle(torch, stream, lambda i: nwc.nwc_read_probe(buf, sink, cus * 8, 1, stream=stream))
    for layout in (0, 1):
        for per_cu in (2, 4, 8, 16):
            groups = cus * per_cu
            with torch.cuda.stream(stream):
                for i in range(3):
                    nwc.nwc_read_probe(buf, sink, groups, layout, stream=stream)
                e0.record(stream)
                for i in range(reps):
                    nwc.nwc_read_probe(buf, sink, groups, layout, stream=stream)
                e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            gbps = PROBE_BYTES / (us * 1e-6) / 1e9
            if best is None or gbps > best["GBps"]:
                best = {"GBps": round(gbps, 1), "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
                        "bytes": PROBE_BYTES, "layout": ("grid-stride", "contiguous per workgroup")[layout],
                        "workgroups": groups, "avg_launch_us": round(us, 2)}
    del buf
    return best


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.model_step:
        model_step(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (a matrix would shard by row "
              "blocks, one blob per GPU, with no cross-GPU reduction at batch 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import decode_gemv_byte_amd as nwc
    import workloads

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    if args.probe_only:
        print(json.dumps({"read_probe": read_probe(torch, nwc, torch.cuda.Stream())}))
        return
    wl = workloads.WORKLOADS[args.workload]
    batch = args.batch or wl.batches[0]
    if not 1 <= batch <= 8192:
        sys.exit("batch must be 1..8192 (above 16: decode + hipBLASLt GEMM)")
    params = {k: v for k, v in (("tile_rows", args.tile_rows), ("max_code_len", args.max_code_len),
                                ("pair_fit", args.pair_fit)) if v}
    if args.code_family == "unary":
        params["code_family"] = 1
        params.setdefault("max_code_len", 12)
    groups_named = [list(g) for g in wl.groups] if wl.groups else [[m.name] for m in wl.matrices]
    tuned, enc_params = None, {m.name: params or None for m in wl.matrices}
    if args.geometry == "tuned":
        if params:
            sys.exit("--geometry tuned chooses the tile rows and length limit itself")
        if batch > 16:
            sys.exit("--geometry tuned covers the fused paths (batch 1..16)")
        from decode_gemv_byte_amd import tune
        tuned = {}
        for g in groups_named:   # layer 0's matrices stand for every layer of the same shape
            r = tune.tune_geometry([workloads.weights(wl.cid, n) for n in g], batch=batch)
            tuned["+".join(g)] = r.as_dict()
            for n in g:
                enc_params[n] = r.params()
            print("[tune] %s: %s" % ("+".join(g), r.as_dict()), file=sys.stderr, flush=True)
    # the step: every layer's groups in order; a key is (layer, matrix name)
    groups = [[(l, n) for n in g] for l in range(wl.layers) for g in groups_named]
    # the dominant launch: the group with the most weights, the first such in
    # step order (layer 0's gate+up in a full step)
    mats = {m.name: m for m in wl.matrices}
    gw = [sum(mats[n].rows * mats[n].cols for (_, n) in g) for g in groups]
    gi = int(np.argmax(gw))
    if args.roofline_only:   # only the dominant launch's matrices are needed
        groups = [groups[gi]]
        gi = 0
    keys = [k for g in groups for k in g]
    want_bf16 = not args.skip_bf16 and not args.roofline_only

    # ---------------------------------------------------------------- setup
    # weights drawn and encoded on the host, matrices in parallel (numpy's
    # generators and the encoder release the interpreter lock)
    t0 = time.time()
    host_blob, info, check, wbf = {}, {}, {}, {}

    def prepare(k):
        l, n = k
        w = workloads.weights(wl.cid, n, layer=l)
        blob = nwc.nwc_encode(w, enc_params[n])
        rng = np.random.default_rng(np.random.SeedSequence([1, l, mats[n].mid]))
        rows = np.unique(np.concatenate([rng.choice(w.shape[0], min(CHECK_ROWS, w.shape[0]), replace=False),
                                         [0, w.shape[0] - 1]]))
        return k, w, blob, (rows, w[rows].copy())

    with ThreadPoolExecutor(max_workers=min(8, host_threads())) as ex:
        for k, w, blob, chk in ex.map(prepare, keys):
            host_blob[k] = blob
            info[k] = nwc.nwc_inspect(blob)
            check[k] = chk
            if want_bf16:
                wbf[k] = torch.from_numpy(w.view(np.int16)).to(dev)
            del w
    enc_s = time.time() - t0
    note("encoded %d matrices in %.1f s" % (len(keys), enc_s))
    # the fused skinny GEMM takes up to 16 X rows, up to 32 with 8-row tiles
    # (matrix cores); more go through the decode + hipBLASLt path
    skinny = batch > 1 and not args.force_prefill and (
        batch <= 16 or (batch <= 32 and all(info[k].tile_rows == 8 for k in keys)))

    def cbytes(k):  # compressed bytes of one GEMV / GEMM: blob + x + y
        return host_blob[k].size + 2 * batch * (info[k].cols + info[k].rows)

    def ubytes(k):
        return 2 * info[k].rows * info[k].cols + 2 * batch * (info[k].cols + info[k].rows)

    bytes_c = sum(cbytes(k) for k in keys)
    bytes_u = sum(ubytes(k) for k in keys)
    gbytes = [sum(cbytes(k) for k in g) for g in groups]
    blob_total = sum(host_blob[k].size for k in keys)
    # (a workload far smaller than the cache, like the 1024x1024 matrix, is
    # launch-bound anyway; 64 copies bound the graphs it needs)
    copies = args.copies or min(64, max(1, int(np.ceil(STREAM_BYTES / blob_total))))

    blobs = [{k: torch.from_numpy(host_blob[k]).to(dev) for k in keys} for _ in range(copies)]
    del host_blob
    xs = {k: torch.from_numpy(workloads.activations(wl.cid, k[1], batch=batch, layer=k[0])).to(dev) for k in keys}
    ys = {k: torch.empty((batch, info[k].rows) if batch > 1 else (info[k].rows,), dtype=torch.bfloat16, device=dev)
          for k in keys}
    stream = torch.cuda.Stream()

    def zeroed(nbytes):
        # workspaces are zero-filled once; every call leaves them zero
        return torch.zeros(max(1, nbytes), dtype=torch.uint8, device=dev)

    if batch == 1:
        gws = [zeroed(nwc.gemv_batched_workspace_size([info[k] for k in g])) for g in groups]
        launches = [[nwc.GemvBatch([info[k] for k in g], [blobs[c][k] for k in g], [xs[k][0] for k in g],
                                   [ys[k] for k in g], gws[i]) for i, g in enumerate(groups)] for c in range(copies)]

        def launch(c, i):
            nwc.nwc_gemv_batched(launches[c][i], stream=stream)
    elif skinny:
        kws = {k: zeroed(nwc.nwc_workspace_size(info[k], batch)) for k in keys}

        def launch(c, i):
            for k in groups[i]:
                nwc.nwc_gemm_skinny(info[k], blobs[c][k], xs[k], ys[k], kws[k], stream=stream)
    else:
        # prefill: each matrix decoded into one shared BF16 workspace, then a
        # hipBLASLt GEMM (the calls run one after another on one stream)
        blas = nwc.Blas()
        pws = torch.empty(max(nwc.nwc_prefill_workspace_size(info[k]) for k in keys), dtype=torch.uint8, device=dev)

        def launch(c, i):
            for k in groups[i]:
                nwc.nwc_gemm_prefill(blas, info[k], blobs[c][k], xs[k], ys[k], pws, stream=stream)

    def step(c):
        for i in range(len(groups)):
            launch(c, i)

    reps = args.roofline_reps
    # the dominant launch alone cycles through its own >= 1 GB of blob
    # copies (one launch's blobs fit the 256 MB Infinity Cache: relaunching
    # the same ones would time the cache, not HBM)
    dcopies = max(copies, int(np.ceil(STREAM_BYTES / gbytes[gi])))
    dblobs = [{k: (blobs[c][k] if c < copies else blobs[0][k].clone()) for k in groups[gi]} for c in range(dcopies)]
    if batch == 1:
        dbatch = [nwc.GemvBatch([info[k] for k in groups[gi]], [dblobs[c][k] for k in groups[gi]],
                                [xs[k][0] for k in groups[gi]], [ys[k] for k in groups[gi]], gws[gi])
                  for c in range(dcopies)]

    def launch_dominant(c):
        if batch == 1:
            nwc.nwc_gemv_batched(dbatch[c], stream=stream)
        elif skinny:
            for k in groups[gi]:
                nwc.nwc_gemm_skinny(info[k], dblobs[c][k], xs[k], ys[k], kws[k], stream=stream)
        else:
            for k in groups[gi]:
                nwc.nwc_gemm_prefill(blas, info[k], dblobs[c][k], xs[k], ys[k], pws, stream=stream)

    def time_dominant():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        settle(torch, stream, lambda i: launch_dominant(i % dcopies))
        with torch.cuda.stream(stream):
            e0.record(stream)
            for i in range(reps):
                launch_dominant(i % dcopies)
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    dom_name = "+".join("%s%s" % (n, "@%d" % l if wl.layers > 1 else "") for (l, n) in groups[gi])
    # the skinny GEMM runs on the matrix cores (k_skinny_mc) from 5 X rows with 8-row tiles
    mc = skinny and batch >= 5 and all(info[k].tile_rows == 8 for k in groups[gi])
    kernel = ("k_gemv via nwc_gemv_batched" if batch == 1 else
              "k_skinny_mc via nwc_gemm_skinny" if mc else
              "k_gemv skinny mode via nwc_gemm_skinny" if skinny else
              "k_gemv decode mode + hipBLASLt GEMM via nwc_gemm_prefill")

    def roofline(us):
        if batch == 1 or skinny:
            a = gbytes[gi] / (us * 1e-6) / 1e9
            return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(a / HBM_PEAK_GBPS, 4),
                    "traffic": (traffic_from_profile(traffic_file(wl.name, [n for (_, n) in groups[gi]]))
                                if batch == 1 and not params and tuned is None else None),
                    "kernel": "%s (%s)" % (kernel, dom_name), "bytes_per_launch": int(gbytes[gi]),
                    "avg_launch_us": round(us, 3), "device_copies_cycled": dcopies,
                    "frac_of_read_probe": (round(a / probe["GBps"], 4) if probe else None)}
        # prefill: the decode writes W' once and the GEMM reads it back, so
        # its bytes are blob + 4 N K + X + Y; past the ridge point the GEMM's
        # flops bound it instead
        g_bytes = sum(info[k].blob_bytes + 4 * info[k].rows * info[k].cols + 2 * batch * (info[k].rows + info[k].cols)
                      for k in groups[gi])
        g_flops = sum(2.0 * batch * info[k].rows * info[k].cols for k in groups[gi])
        if g_flops / g_bytes > MFMA_BF16_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):
            a = g_flops / (us * 1e-6) / 1e12
            return {"bound": "mfma", "achieved": round(a, 1), "peak": MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(a / MFMA_BF16_TFLOPS, 4), "traffic": None,
                    "kernel": "%s (%s)" % (kernel, dom_name), "flops_per_launch": g_flops,
                    "avg_launch_us": round(us, 3)}
        a = g_bytes / (us * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBPS, 4), "traffic": None,
                "kernel": "%s (%s)" % (kernel, dom_name), "bytes_per_launch": int(g_bytes),
                "avg_launch_us": round(us, 3)}

    probe = None
    if args.roofline_only:
        us = time_dominant()
        print(json.dumps({"roofline": roofline(us), "config": {"workload": wl.name, "batch": batch}}))
        return

    # correctness guard (not timed): sampled rows of every output against an
    # FP64 product of the same BF16 values, after one eager step and again
    # after the timed graph replays
    def verify(when):
        for k in keys:
            rows, wr = check[k]
            wf = torch.from_numpy(wr.view(np.int16)).view(torch.bfloat16).double()
            xf = xs[k].cpu().view(torch.bfloat16).double()                      # [batch, K]
            ref = (xf @ wf.T).numpy()
            a = (xf.abs() @ wf.abs().T).numpy()
            got = ys[k].reshape(batch, -1).cpu().double().numpy()[:, rows]
            if not np.all(np.abs(got - ref) <= 2.0 ** -10 * a + 2.0 ** -8 * np.abs(ref)):
                print("bench: %s outside tolerance %s" % (k, when), file=sys.stderr)
                sys.exit(1)

    with torch.cuda.stream(stream):
        step(0)
    torch.cuda.synchronize()
    verify("after an eager step")
    note("eager step verified (%d copies on the device)" % copies)

    graphs = None
    if not args.no_graph:
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(c)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(n, start):
        for i in range(n):
            c = (start + i) % copies
            with torch.cuda.stream(stream):
                if graphs is not None:
                    graphs[c].replay()
                else:
                    step(c)

    # --------------------------------------------------------------- timed
    settle(torch, stream, lambda i: run(1, i))
    run(args.warmup, 0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    e0.record(stream)
    run(args.steps, args.warmup)
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_start
    ms_per_step = e0.elapsed_time(e1) / args.steps
    verify("after the timed steps")
    value = bytes_c / (ms_per_step * 1e-3) / 1e9
    value_u = bytes_u / (ms_per_step * 1e-3) / 1e9
    note("timed %d steps: %.4f ms per step" % (args.steps, ms_per_step))
    dom_us = time_dominant()
    probe = read_probe(torch, nwc, stream)
    note("dominant launch %.2f us; read probe %.0f GB/s" % (dom_us, probe["GBps"]))

    # every GEMV of a one-layer batch-1 step in a single launch (they read
    # independent activations here): what the launch boundaries cost (one
    # launch takes one tile height)
    single = None
    if batch == 1 and wl.layers == 1 and len(groups) > 1 and len({info[k].tile_rows for k in keys}) == 1:
        iws = zeroed(nwc.gemv_batched_workspace_size([info[k] for k in keys]))
        allb = [nwc.GemvBatch([info[k] for k in keys], [blobs[c][k] for k in keys], [xs[k][0] for k in keys],
                              [ys[k] for k in keys], iws) for c in range(copies)]
        settle(torch, stream, lambda i: nwc.nwc_gemv_batched(allb[i % copies], stream=stream))
        with torch.cuda.stream(stream):
            e0.record(stream)
            for i in range(reps):
                nwc.nwc_gemv_batched(allb[i % copies], stream=stream)
            e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        single = {"us": round(us, 3), "compressed_GBps": round(bytes_c / (us * 1e-6) / 1e9, 1)}

    # -------------------------------------------- standalone decode (A5)
    # every matrix of the step decoded to BF16 in HBM; bytes = blob read +
    # 2 bytes per weight written
    decode = None
    if batch == 1:
        wout = {k: torch.empty((info[k].rows, info[k].cols), dtype=torch.int16, device=dev) for k in keys}

        # all matrices in one launch when they fit one (up to 8, one geometry)
        one = len(keys) <= 8 and len({info[k].tile_rows for k in keys}) == 1
        dbatch = [nwc.DecodeBatch([info[k] for k in keys], [blobs[c][k] for k in keys], [wout[k] for k in keys])
                  for c in range(copies)] if one else None

        def step_decode(c):
            if one:
                nwc.nwc_decode_batched(dbatch[c], stream=stream)
                return
            for k in keys:
                nwc.nwc_decode(info[k], blobs[c][k], wout[k], stream=stream)
        dgraphs = []
        for c in range(copies if graphs is not None else 0):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step_decode(c)
            dgraphs.append(g)
        torch.cuda.synchronize()

        def decode_once(i):
            with torch.cuda.stream(stream):
                dgraphs[i % copies].replay() if dgraphs else step_decode(i % copies)
        settle(torch, stream, decode_once)
        for i in range(args.warmup):
            decode_once(i)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            with torch.cuda.stream(stream):
                dgraphs[i % copies].replay() if dgraphs else step_decode(i % copies)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_d = e0.elapsed_time(e1) / args.steps
        moved = blob_total + sum(2 * info[k].rows * info[k].cols for k in keys)
        decode = {"launches": 1 if one else len(keys), "ms_per_step": round(ms_d, 5),
                  "GBps_moved": round(moved / (ms_d * 1e-3) / 1e9, 1),
                  "bytes_moved": int(moved), "pct_hbm_peak": round(100.0 * moved / (ms_d * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)}
        del wout, dgraphs, dbatch

    # ------------------------------- embedding lookup from a tied LM head
    # rows by token id straight from the compressed matrix, against torch's
    # index_select on the BF16 weights (one launch each, HIP events)
    gather = None
    if args.workload == 5:
        k = keys[0]
        g_rng = np.random.default_rng(7)
        gather = {}
        for n_ids in (1, 16, 256):
            ids = torch.from_numpy(g_rng.integers(0, info[k].rows, n_ids).astype(np.int32)).to(dev)
            gout = torch.empty((n_ids, info[k].cols), dtype=torch.int16, device=dev)
            ge0, ge1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            settle(torch, stream, lambda i: nwc.nwc_gather_rows(info[k], blobs[i % copies][k], ids, gout, stream=stream))
            with torch.cuda.stream(stream):
                ge0.record(stream)
                for i in range(50):
                    nwc.nwc_gather_rows(info[k], blobs[i % copies][k], ids, gout, stream=stream)
                ge1.record(stream)
            torch.cuda.synchronize()
            entry = {"us": round(ge0.elapsed_time(ge1) * 1e3 / 50, 3)}
            if want_bf16:
                ids64 = ids.long()
                settle(torch, stream, lambda i: torch.index_select(wbf[k], 0, ids64))
                with torch.cuda.stream(stream):
                    ge0.record(stream)
                    for i in range(50):
                        torch.index_select(wbf[k], 0, ids64)
                    ge1.record(stream)
                torch.cuda.synchronize()
                entry["torch_index_select_us"] = round(ge0.elapsed_time(ge1) * 1e3 / 50, 3)
            gather["rows_%d" % n_ids] = entry

    # ------------------------------------------------ plain BF16 comparators
    bf16 = None
    if want_bf16:
        bf16 = bf16_comparators(torch, nwc, args, keys, info, wbf, xs, ys, batch, bytes_u, ms_per_step, stream,
                                zeroed, groups[gi], dom_us, probe)
        wbf.clear()

    # ------------------------------------------------------- CPU baseline
    note("comparators and standalone decode done")
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, keys, info, batch, args.cpu_seconds, args.pair_fit or DEFAULT_PAIR_FIT,
                           1 if args.code_family == "unary" else 0)

    out = {
        "metric": "fused decode-GEMV GB/s (compressed + uncompressed-equiv), % HBM peak, batch 1",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": SETTLE_MS,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.layers,
                   "matrices": {m.name: [m.rows, m.cols] for m in wl.matrices}, "batch": batch,
                   "launch_order": groups_named, "launches_per_step": len(groups),
                   "device_copies": copies, "hip_graph": graphs is not None, "output": "bf16",
                   "encoder": ({"tuned": tuned} if tuned else params or "default"),
                   "path": ("fused decode-GEMV" if batch == 1 else "fused skinny decode-GEMM" if skinny
                            else "decode to BF16 + hipBLASLt GEMM")},
        "compressed_GBps": round(value, 1),
        "uncompressed_equiv_GBps": round(value_u, 1),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "bytes_per_step": {"compressed": int(bytes_c), "uncompressed": int(bytes_u)},
        "bf16_gemv": bf16,
        "single_launch_all_gemvs": single,
        "standalone_decode": decode,
        "embedding_gather": gather,
        "read_probe": probe,
        "pct_read_probe": round(100.0 * value / probe["GBps"], 2),
        "roofline": roofline(dom_us),
        "cpu_baseline": cpu,
        "wall_s": round(t_wall, 3),
        "encode_s": round(enc_s, 2),
    }
    print(json.dumps(out))


def bf16_comparators(torch, nwc, args, keys, info, wbf, xs, ys, batch, bytes_u, ms_per_step, stream, zeroed,
                     dom_keys, dom_us, probe):
    """The same GEMVs reading plain BF16 weights: our kernel with the same
    skeleton (batch 1) and the vendor library's product (torch.mv /
    F.linear), same matrices, same launch order, graph-captured, cycling
    enough device copies to stream from HBM.  At batch 1 also the dominant
    launch's matrices alone through our comparator (one launch each, copies
    cycled past the Infinity Cache), against the read probe."""
    ub = sum(2 * info[k].rows * info[k].cols for k in keys)
    bcopies = max(1, int(np.ceil(STREAM_BYTES / ub)))
    wdev = [{k: (wbf[k] if c == 0 else wbf[k].clone()) for k in keys} for c in range(bcopies)]
    yb = {k: torch.empty_like(ys[k]) for k in keys}
    wsb = {k: zeroed(nwc.nwc_bf16_workspace_size(info[k].rows, info[k].cols)) for k in keys}

    def graphs_of(fn):
        with torch.cuda.stream(stream):
            fn(0)
        torch.cuda.synchronize()
        out = []
        for c in range(bcopies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                fn(c)
            out.append(g)
        torch.cuda.synchronize()
        return out

    def rep_timed(gr):
        settle(torch, stream, lambda i: gr[i % bcopies].replay())
        for i in range(args.warmup):
            with torch.cuda.stream(stream):
                gr[i % bcopies].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            with torch.cuda.stream(stream):
                gr[i % bcopies].replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    res = {}
    if batch == 1:
        def step_ours(c):
            for k in keys:
                nwc.nwc_gemv_bf16(wdev[c][k], xs[k][0], yb[k], wsb[k], stream=stream)
        ms_b = rep_timed(graphs_of(step_ours))
        res.update(ms_per_step=round(ms_b, 5), GBps=round(bytes_u / (ms_b * 1e-3) / 1e9, 1),
                   speedup_fused_vs_bf16=round(ms_b / ms_per_step, 3))
    wt = [{k: wdev[c][k].view(torch.bfloat16) for k in keys} for c in range(bcopies)]
    xt = {k: xs[k].view(torch.bfloat16) for k in keys}
    yt = {k: torch.empty(ys[k].shape, dtype=torch.bfloat16, device=ys[k].device) for k in keys}

    def step_torch(c):
        for k in keys:
            if batch == 1:
                torch.mv(wt[c][k], xt[k][0], out=yt[k])
            else:
                torch.nn.functional.linear(xt[k], wt[c][k], out=yt[k])
    ms_t = rep_timed(graphs_of(step_torch))
    res["torch"] = dict(op="torch.mv" if batch == 1 else "torch.nn.functional.linear",
                        ms_per_step=round(ms_t, 5), GBps=round(bytes_u / (ms_t * 1e-3) / 1e9, 1),
                        speedup_fused_vs_torch=round(ms_t / ms_per_step, 3))
    if batch == 1:
        # the dominant launch's matrices: our comparator alone, copies cycled
        db = sum(2 * info[k].rows * info[k].cols for k in dom_keys)
        dcopies = max(2, int(np.ceil(STREAM_BYTES / db)))
        dw = [{k: (wbf[k] if c == 0 else wbf[k].clone()) for k in dom_keys} for c in range(dcopies)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = args.roofline_reps

        def bf16_dom(i):
            for k in dom_keys:
                nwc.nwc_gemv_bf16(dw[i % dcopies][k], xs[k][0], yb[k], wsb[k], stream=stream)
        settle(torch, stream, bf16_dom)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for i in range(reps):
                bf16_dom(i)
            e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        moved = sum(2 * info[k].rows * info[k].cols + 2 * (info[k].rows + info[k].cols) for k in dom_keys)
        gbps = moved / (us * 1e-6) / 1e9
        res["dominant_launch_matrices"] = {
            "matrices": ["%s@%d" % (n, l) for (l, n) in dom_keys], "launches": len(dom_keys),
            "us": round(us, 3), "GBps": round(gbps, 1), "frac_of_read_probe": round(gbps / probe["GBps"], 4),
            "speedup_fused_vs_bf16": round(us / dom_us, 3)}
        del dw
    return res


def cpu_baseline(wl, keys, info, batch, seconds, pair_fit, family=0):
    """The oracle (plain C: bit-serial decode and FP64 GEMV/GEMM) on a bounded
    sample of the workload: 256-row blocks of its matrices taken round robin
    (each matrix's first rows first), each encoded by the oracle with the
    library blob's geometry, code length limit and 6-bit cap (encoding is not
    timed: the GPU figure excludes it too), then decoded and multiplied.  The
    blocks are timed on one thread until about `seconds` of work, then the
    same blocks again through a pool of all the host threads this process may
    use (wall clock; the oracle's C calls release the interpreter lock).
    Rate in compressed bytes (blob + x + y) per second, the same definition as
    the GPU figure."""
    import oracle
    import workloads

    nb = 256
    threads = host_threads()

    def sample(i):
        layer, name = keys[i % len(keys)]
        li = info[(layer, name)]
        r0 = (i // len(keys)) * nb % li.rows
        sub = workloads.weights(wl.cid, name, layer=layer, rows=slice(r0, min(r0 + nb, li.rows)))
        blob = oracle.encode(sub, li.tile_rows, li.tile_cols, li.chunks_per_tile, li.max_code_len, pair_fit, family)
        x = workloads.activations(wl.cid, name, batch=batch, layer=layer)
        return blob, x, blob.size + 2 * batch * (sub.shape[1] + sub.shape[0])

    def work(item):
        blob, x, _ = item
        wd = oracle.decode(blob)
        if batch == 1:
            oracle.gemv(wd, x[0])
        else:
            oracle.gemm(wd, x)

    # one thread: blocks prepared `threads` at a time, worked until `seconds`
    items, t_one = [], 0.0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while t_one < seconds and len(items) < 2000:
            fresh = list(ex.map(sample, range(len(items), len(items) + threads)))
            for it in fresh:
                t = time.perf_counter()
                work(it)
                t_one += time.perf_counter() - t
                items.append(it)
                if t_one >= seconds:
                    break
        # all threads: the same blocks through the pool
        t = time.perf_counter()
        list(ex.map(work, items))
        t_all = time.perf_counter() - t
    moved = float(sum(it[2] for it in items))
    return {"value": round(moved / t_all / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(), "logical_cpus_visible": os.cpu_count(),
            "single_thread": {"value": round(moved / t_one / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "seconds": round(t_one, 2)},
            "sample": "%d row blocks of 256 rows from the workload's matrices (round robin), oracle decode + FP64 "
                      "%s: %.1f s on one thread, then %.2f s wall on %d threads"
                      % (len(items), "GEMV" if batch == 1 else "GEMM", t_one, t_all, threads)}


if __name__ == "__main__":
    main()
