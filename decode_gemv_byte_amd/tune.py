"""Per-shape geometry tuning: choose the tile geometry of a blob by timing the
fused kernels on the GPU at hand.

The format leaves the tile geometry to the encoder (rows per tile, the code
length limit).  Which one is fastest depends on the matrix shape, the batch
and the GPU: a shorter tile gives a launch more, smaller work items (less
idle time at the start and end of a launch) at the cost of a few more bytes
of chunk and offset tables; the length limit trades code efficiency against
the decoder's two-code fallback.  The pages fix the code per tensor and use
one block shape, 8 rows by 512 columns, for every matrix ("NWC -- Neural
Weight Compression", How it works, bullet "Fused kernel"); this module
makes the choice per shape, empirically, for the matrices that one launch
processes together.

Every candidate is encoded on the host, checked to decode back to the exact
input bits on the GPU, and timed as a captured graph of launches that cycle
through enough device copies that each launch streams its blob from HBM
(not from the last-level cache).  Nothing here changes a blob's meaning:
every geometry decodes to the same weights.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple, Union

import numpy as np

from . import (GemvBatch, NwcError, nwc_decode, nwc_encode, nwc_gemm_skinny, nwc_gemv, nwc_gemv_batched,
               nwc_inspect, nwc_workspace_size)

# (tile_rows, max_code_len): the tile heights the fused kernels run natively
# at the default length limit, one step above it, and the 6-bit limit under
# which every decode step reads two codes with one lookup (about 0.4 bit per
# weight more; only for tensors with at most 64 distinct exponents, else the
# library rejects the candidate)
DEFAULT_CANDIDATES: Tuple[Tuple[int, int], ...] = ((4, 8), (8, 8), (16, 8), (32, 8), (8, 9), (4, 6), (8, 6))
STREAM_BYTES = 768 << 20   # device copies cycled per timing: well above the last-level cache
MAX_COPIES = 32
SETTLE_MS = 50.0           # GPU time a candidate runs before it is timed


@dataclass
class Candidate:
    tile_rows: int
    max_code_len: int
    blob_bytes: int
    us: float                      # average duration of one launch (or of the batch's calls); inf if
                                   # the library rejects this geometry for these matrices

    def params(self) -> Dict[str, int]:
        return {"tile_rows": self.tile_rows, "max_code_len": self.max_code_len}


@dataclass
class TuneResult:
    best: Candidate
    candidates: List[Candidate] = field(default_factory=list)
    batch: int = 1

    def params(self) -> Dict[str, int]:
        return self.best.params()

    def as_dict(self) -> dict:
        return {"batch": self.batch, "best": self.best.params(),
                "candidates": [{"tile_rows": c.tile_rows, "max_code_len": c.max_code_len,
                                "blob_bytes": c.blob_bytes, "us": round(c.us, 3) if c.us != float("inf") else None}
                               for c in self.candidates]}


def check_candidates(candidates) -> List[Tuple[int, int]]:
    """Validate (tile_rows, max_code_len) pairs: tile_rows a power of two in
    1..64, max_code_len 6..12 (what the encoder accepts)."""
    out = []
    for c in candidates:
        tr, lmax = (int(c[0]), int(c[1]))
        if tr < 1 or tr > 64 or tr & (tr - 1):
            raise ValueError("tile_rows must be a power of two in 1..64, got %d" % tr)
        if not 6 <= lmax <= 12:
            raise ValueError("max_code_len must be in 6..12, got %d" % lmax)
        if (tr, lmax) not in out:
            out.append((tr, lmax))
    if not out:
        raise ValueError("no candidates")
    return out


def pick(cands: Sequence[Candidate], size_slack: float = 0.0) -> Candidate:
    """The fastest candidate; with size_slack > 0, the smallest blob among
    those within (1 + size_slack) of the fastest time."""
    fastest = min(cands, key=lambda c: c.us)
    near = [c for c in cands if c.us <= fastest.us * (1.0 + size_slack)]
    return min(near, key=lambda c: (c.blob_bytes, c.us))


def _time_candidate(ws_bits, blobs_host, batch, reps, device):
    import torch

    infos = [nwc_inspect(b) for b in blobs_host]
    total = sum(b.size for b in blobs_host)
    copies = max(2, min(MAX_COPIES, -(-STREAM_BYTES // max(1, total))))
    dev_blobs = [[torch.from_numpy(b).to(device) for b in blobs_host] for _ in range(copies)]
    # the blob must decode to the input bits exactly before it is timed
    for w, info, blob in zip(ws_bits, infos, dev_blobs[0]):
        ld = (int(info.cols) + 7) // 8 * 8
        out = torch.empty((int(info.rows), ld), dtype=torch.int16, device=device)
        nwc_decode(info, blob, out, ld)
        if not torch.equal(out[:, :int(info.cols)].cpu(), torch.from_numpy(w.view(np.int16))):
            raise RuntimeError("a candidate blob does not decode to its input")
        del out
    g = torch.Generator(device="cpu").manual_seed(7)
    xs = [torch.randn((batch, int(i.cols)), generator=g).to(torch.bfloat16).to(device) for i in infos]
    ys = [torch.empty((batch, int(i.rows)), dtype=torch.bfloat16, device=device) for i in infos]
    stream = torch.cuda.Stream(device=device)
    if batch == 1 and len(infos) == 1:
        ws = torch.zeros(max(1, nwc_workspace_size(infos[0], 1)), dtype=torch.uint8, device=device)

        def launch(c):
            nwc_gemv(infos[0], dev_blobs[c][0], xs[0][0], ys[0][0], ws, stream=stream)
    elif batch == 1:
        ws = torch.zeros(max(1, sum(nwc_workspace_size(i, 1) for i in infos)), dtype=torch.uint8, device=device)
        calls = [GemvBatch(infos, dev_blobs[c], [x[0] for x in xs], [y[0] for y in ys], ws) for c in range(copies)]

        def launch(c):
            nwc_gemv_batched(calls[c], stream=stream)
    else:
        wss = [torch.zeros(max(1, nwc_workspace_size(i, batch)), dtype=torch.uint8, device=device) for i in infos]

        def launch(c):
            for i, info in enumerate(infos):
                nwc_gemm_skinny(info, dev_blobs[c][i], xs[i].view(torch.int16), ys[i], wss[i], stream=stream)
    with torch.cuda.stream(stream):
        for c in range(copies):   # eager once: builds any state before capture
            launch(c)
    torch.cuda.synchronize(device)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for c in range(copies):
            launch(c)
    rounds = max(1, -(-reps // copies))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # replays until the GPU has run this candidate for SETTLE_MS: a GPU left
    # idle (here, while the host encoded the candidate) runs its first
    # milliseconds of load slower, which would favour later candidates
    settled, n = 0.0, 1
    while settled < SETTLE_MS:
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(n):
                graph.replay()
            e1.record(stream)
        torch.cuda.synchronize(device)
        settled += e0.elapsed_time(e1)
        n = min(2 * n, 1024)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(rounds):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize(device)
    us = e0.elapsed_time(e1) * 1e3 / (rounds * copies)
    del graph
    return us


def tune_geometry(w: Union[np.ndarray, Sequence[np.ndarray]], batch: int = 1, candidates=DEFAULT_CANDIDATES,
                  reps: int = 100, size_slack: float = 0.0, device=None) -> TuneResult:
    """Time every candidate geometry for the matrices that one launch
    processes together (w: one uint16 BF16-bit matrix, or a list sharing a
    launch: at batch 1 they run as one nwc_gemv_batched call, above it as
    one nwc_gemm_skinny call each) and return the fastest (see pick).  A
    geometry the library rejects for these matrices (NwcError) is kept in
    the table with an infinite time; if every candidate is rejected the last
    error is raised."""
    import torch

    mats = [w] if isinstance(w, np.ndarray) else list(w)
    if not mats:
        raise ValueError("no matrices")
    for m in mats:
        if m.dtype != np.uint16 or m.ndim != 2:
            raise ValueError("expected 2-D uint16 BF16 bit patterns")
    if not 1 <= batch <= 32:
        raise ValueError("batch must be 1..32 (nwc_gemv_batched at 1, nwc_gemm_skinny above)")
    if batch == 1 and len(mats) > 8:
        raise ValueError("at most 8 matrices share one launch")
    device = torch.device(device or "cuda")
    res, err = [], None
    for tr, lmax in check_candidates(candidates):
        try:
            blobs = [nwc_encode(m, {"tile_rows": tr, "max_code_len": lmax}) for m in mats]
        except NwcError as e:       # e.g. more distinct exponents than a short limit codes
            res.append(Candidate(tr, lmax, 0, float("inf")))
            err = e
            continue
        try:
            us = _time_candidate(mats, blobs, batch, reps, device)
        except NwcError as e:
            us, err = float("inf"), e
        res.append(Candidate(tr, lmax, int(sum(b.size for b in blobs)), us))
    if all(c.us == float("inf") for c in res):
        raise err
    return TuneResult(pick([c for c in res if c.us != float("inf")], size_slack), res, batch)
