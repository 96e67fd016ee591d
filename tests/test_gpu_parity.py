"""GPU parity of libnwc's HIP kernels against the CPU oracle (MI355X only).

Bars:
* decode: bit-exact against the original BF16 bits;
* GEMV / skinny GEMM: per output |y - y_oracle| <= 2^-10 * sum|w x| (FP32
  output), plus 2^-8 * |y_oracle| for BF16 output (one final rounding), with
  y_oracle and sum|w x| from the oracle's FP64 products;
* repeated calls give bitwise-identical results.
Small cases compare every output here; the full-size workloads are checked
row by row in test_gpu_configs.py (the prefill path, beyond the skinny
batches, on sampled rows below).
"""
import functools
import os
import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
import decode_gemv_byte_amd as nwc  # noqa: E402

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _say(msg):
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class Blob:
    def __init__(self, w: np.ndarray, params=None):
        self.w = w
        self.host = nwc.nwc_encode(w, params)
        self.info = nwc.nwc_inspect(self.host)
        self.dev = dev(self.host)

    def ws(self, batch=1):
        # zero-filled: the fused batch-1 path keeps counters there
        return torch.zeros(nwc.nwc_workspace_size(self.info, batch), dtype=torch.uint8, device="cuda")


@functools.lru_cache(maxsize=None)
def _w(cid, name, layer=0):
    return workloads.weights(cid, name, layer=layer)


def _check_y(y_gpu, y_ref, a_ref, out_f32, what):
    y_gpu = np.asarray(y_gpu, np.float64)
    tol = 2.0 ** -10 * a_ref
    if not out_f32:
        tol = tol + 2.0 ** -8 * np.abs(y_ref)
    err = np.abs(y_gpu - y_ref)
    bad = np.flatnonzero(~(err <= tol))
    assert bad.size == 0, "%s: %d/%d outside tolerance, first %s: got %r want %r tol %r" % (
        what, bad.size, err.size, bad[:5], y_gpu[bad[:5]], y_ref[bad[:5]], tol[bad[:5]])


def _to_f64(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def _gemv(blob: Blob, x: np.ndarray, out_f32: bool):
    xd = dev(x)
    y = torch.empty(blob.info.rows, dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    nwc.nwc_gemv(blob.info, blob.dev, xd, y, blob.ws())
    torch.cuda.synchronize()
    return y


# ----------------------------------------------------------------- decode --

def _special(name):
    rng = np.random.default_rng(5)
    return {
        "cfg1": lambda: _w(1, "w"),
        "all_patterns": workloads.all_patterns,
        "127x1001": lambda: workloads.gaussian_bits((127, 1001), 0.02, 4),
        "1x1": lambda: workloads.gaussian_bits((1, 1), 0.02, 1),
        "1000x256": lambda: workloads.gaussian_bits((1000, 256), 0.02, 7),
        "nan_payloads": lambda: (0x7F80 | rng.integers(1, 128, (33, 64)) |
                                 (rng.integers(0, 2, (33, 64)) << 15)).astype(np.uint16),
        "subnormal": lambda: (rng.integers(1, 128, (48, 72)) | (rng.integers(0, 2, (48, 72)) << 15)).astype(np.uint16),
        "one_symbol": lambda: (0x3C00 | rng.integers(0, 128, (50, 64))).astype(np.uint16),
        "random_bits": lambda: workloads.random_bits((300, 264), 6),
        "wide_odd": lambda: workloads.gaussian_bits((40, 3000), 0.05, 8),
        "8x512": lambda: workloads.gaussian_bits((8, 512), 0.02, 9),
        "3000x512": lambda: workloads.gaussian_bits((3000, 512), 0.02, 10),
        "20x40960": lambda: workloads.gaussian_bits((20, 40960), 0.02, 12),
    }[name]()


DECODE_CASES = [("cfg1", None), ("cfg1", dict(tile_rows=16)), ("cfg1", dict(tile_rows=32)),
                ("cfg1", dict(tile_rows=5, tile_cols=24, chunks_per_tile=3, max_code_len=11)),
                ("all_patterns", None), ("127x1001", None), ("1x1", None), ("1000x256", None),
                ("nan_payloads", None), ("subnormal", None), ("one_symbol", None), ("random_bits", None),
                ("wide_odd", None), ("wide_odd", dict(tile_rows=3, tile_cols=7, chunks_per_tile=7, max_code_len=10)),
                ("cfg1", dict(max_code_len=12)), ("all_patterns", dict(max_code_len=12)),
                ("cfg1", dict(tile_rows=4)), ("1000x256", dict(tile_rows=4)),
                # code limits below 8: at 6 the fused decode never takes a second lookup
                ("cfg1", dict(max_code_len=6)), ("cfg1", dict(max_code_len=7)), ("subnormal", dict(max_code_len=6)),
                ("1000x256", dict(tile_rows=4, max_code_len=6)), ("cfg1", dict(tile_rows=16, max_code_len=6)),
                ("cfg1", dict(tile_rows=32, max_code_len=6)), ("127x1001", dict(max_code_len=6))]


@pytest.mark.parametrize("name,params", DECODE_CASES)
def test_decode_bit_exact(name, params):
    w = _special(name)
    _say("decode %s %s %s" % (name, w.shape, params))
    b = Blob(w, params)
    out = torch.full(w.shape, 0x5A5A, dtype=torch.int16, device="cuda")
    nwc.nwc_decode(b.info, b.dev, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, w)


def test_decode_padded_leading_dimension():
    w = _special("127x1001")
    b = Blob(w)
    for ld in (1008, 1013):           # vector path (ld % 8 == 0) and scalar path
        _say("decode ld=%d" % ld)
        out = torch.full((w.shape[0], ld), 0x1234, dtype=torch.int16, device="cuda")
        nwc.nwc_decode(b.info, b.dev, out, ld=ld)
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint16)
        assert np.array_equal(got[:, :1001], w)
        assert np.all(got[:, 1001:] == 0x1234)     # nothing written past the row


def test_decode_batched_equals_originals():
    # the seven matrices of one layer in one launch, one of them into a wider
    # output (ld > cols): every weight back bit-exactly, nothing written past
    # a row
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    ws = [_w(2, n) for n in names]
    blobs = [Blob(w) for w in ws]
    outs = []
    for i, w in enumerate(ws):
        ld = w.shape[1] + (8 if i == 2 else 0)
        outs.append(torch.full((w.shape[0], ld), 0x1234, dtype=torch.int16, device="cuda"))
    _say("decode_batched 7 matrices")
    nwc.nwc_decode_batched(nwc.DecodeBatch([b.info for b in blobs], [b.dev for b in blobs], outs))
    torch.cuda.synchronize()
    for w, out, n in zip(ws, outs, names):
        got = out.cpu().numpy().view(np.uint16)
        assert np.array_equal(got[:, :w.shape[1]], w), n
        assert np.all(got[:, w.shape[1]:] == 0x1234), n


def test_decode_oracle_written_blob():
    # the GPU decoder follows the format, not just the library's encoder
    w = _w(1, "w")
    host = oracle.encode(w, 8, 512, 64, 12)
    info = nwc.nwc_inspect(host)
    out = torch.empty(w.shape, dtype=torch.int16, device="cuda")
    nwc.nwc_decode(info, dev(host), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), w)


# ------------------------------------------------------------------- GEMV --

GEMV_CASES = [("cfg1", None), ("cfg1", dict(tile_rows=16)), ("cfg1", dict(tile_rows=32)),
              ("cfg1", dict(tile_rows=5, tile_cols=24, chunks_per_tile=3, max_code_len=11)),
              ("127x1001", None), ("1x1", None), ("1000x256", None), ("subnormal", None),
              ("one_symbol", None), ("wide_odd", None), ("8x512", None), ("3000x512", None),
              ("20x40960", None), ("20x40960", dict(tile_rows=16)),
              ("cfg1", dict(max_code_len=12)), ("3000x512", dict(max_code_len=12)),
              ("cfg1", dict(tile_rows=4)), ("3000x512", dict(tile_rows=4)), ("20x40960", dict(tile_rows=4)),
              ("cfg1", dict(max_code_len=6)), ("cfg1", dict(max_code_len=7)), ("3000x512", dict(max_code_len=6)),
              ("20x40960", dict(tile_rows=4, max_code_len=6)), ("20x40960", dict(tile_rows=32, max_code_len=6)),
              ("1000x256", dict(tile_rows=16, max_code_len=6)), ("127x1001", dict(max_code_len=6))]


@pytest.mark.parametrize("out_f32", [False, True])
@pytest.mark.parametrize("name,params", GEMV_CASES)
def test_gemv_small(name, params, out_f32):
    w = _special(name)
    x = workloads.gaussian_bits((w.shape[1],), 1.0, 11)
    _say("gemv %s %s %s f32=%s" % (name, w.shape, params, out_f32))
    b = Blob(w, params)
    y = _gemv(b, x, out_f32)
    y_ref, a_ref = oracle.gemv(w, x)
    _check_y(_to_f64(y), y_ref, a_ref, out_f32, name)


def test_gemv_subnormal_products_kept():
    # every weight subnormal and x = 1: FP32 keeps the exact sums (no flush)
    rng = np.random.default_rng(3)
    w = rng.integers(1, 128, (64, 512)).astype(np.uint16)
    x = np.full(512, 0x3F80, np.uint16)
    b = Blob(w)
    y = _gemv(b, x, True)
    y_ref, a_ref = oracle.gemv(w, x)
    assert np.all(y_ref > 0)
    _check_y(_to_f64(y), y_ref, a_ref, True, "subnormal")


def test_gemv_workspace_reused_across_shapes():
    # one workspace, sized for the largest call, serves calls of any size in
    # stream order: each call leaves its counters at zero for the next
    big, small = Blob(_special("3000x512")), Blob(_special("20x40960"))
    ws = torch.zeros(max(nwc.nwc_workspace_size(big.info, 1), nwc.nwc_workspace_size(small.info, 1)),
                     dtype=torch.uint8, device="cuda")
    for b in (big, small, big, small):
        x = workloads.gaussian_bits((b.info.cols,), 1.0, 13)
        y = torch.empty(b.info.rows, dtype=torch.float32, device="cuda")
        _say("gemv reuse %dx%d" % (b.info.rows, b.info.cols))
        nwc.nwc_gemv(b.info, b.dev, dev(x), y, ws)
        torch.cuda.synchronize()
        y_ref, a_ref = oracle.gemv(b.w, x)
        _check_y(_to_f64(y), y_ref, a_ref, True, "reuse")
        assert _counters_zero([b], ws)


def test_gemv_deterministic():
    w = _w(2, "q")
    x = workloads.activations(2, "q")[0]
    b = Blob(w)
    y1 = _gemv(b, x, True).cpu().numpy()
    y2 = _gemv(b, x, True).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "gate", "up", "down"])
def test_gemv_qwen3_4b_layer_full(name):
    w = _w(2, name)
    x = workloads.activations(2, name)[0]
    _say("gemv workload 2 %s %s" % (name, w.shape))
    b = Blob(w)
    y_ref, a_ref = oracle.gemv(w, x)
    for out_f32 in (False, True):
        _check_y(_to_f64(_gemv(b, x, out_f32)), y_ref, a_ref, out_f32, name)


def _batched_ws(blobs):
    return torch.zeros(nwc.gemv_batched_workspace_size([b.info for b in blobs]), dtype=torch.uint8, device="cuda")


def _counters_zero(blobs, ws):
    """Every call leaves its workspace (counters and partial sums) all zero."""
    n = sum(nwc.nwc_workspace_size(b.info, 1) for b in blobs)
    return int(ws[:n].count_nonzero()) == 0


def test_gemv_batched_seven_matrices_and_repeats():
    # the whole layer in one launch: every y within the bound, the workspace
    # left zero, and the same call twice gives the same bits
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    blobs = [Blob(_w(2, n)) for n in names]
    xs = [dev(workloads.activations(2, n)[0]) for n in names]
    for out_f32 in (False, True):
        dt = torch.float32 if out_f32 else torch.bfloat16
        ys = [torch.empty(b.info.rows, dtype=dt, device="cuda") for b in blobs]
        ys2 = [torch.empty_like(y) for y in ys]
        ws = _batched_ws(blobs)
        for out in (ys, ys2):
            batch = nwc.GemvBatch([b.info for b in blobs], [b.dev for b in blobs], xs, out, ws)
            _say("gemv_batched 7 matrices f32=%s" % out_f32)
            nwc.nwc_gemv_batched(batch)
            torch.cuda.synchronize()
            assert _counters_zero(blobs, ws)
        for b, x, y, y2, n in zip(blobs, xs, ys, ys2, names):
            iv = torch.int32 if out_f32 else torch.int16
            assert torch.equal(y.view(iv), y2.view(iv)), n
            y_ref, a_ref = oracle.gemv(b.w, x.cpu().numpy())
            _check_y(_to_f64(y), y_ref, a_ref, out_f32, n)


def test_gemv_batched_mixed_shapes_and_edges():
    ws = [workloads.gaussian_bits((1000, 256), 0.02, 1), workloads.gaussian_bits((37, 1024), 0.05, 2),
          workloads.gaussian_bits((300, 2048), 0.01, 3)]
    blobs = [Blob(w) for w in ws]
    xs = [dev(workloads.gaussian_bits((w.shape[1],), 1.0, 5 + i)) for i, w in enumerate(ws)]
    ys = [torch.empty(w.shape[0], dtype=torch.float32, device="cuda") for w in ws]
    wsp = _batched_ws(blobs)
    nwc.nwc_gemv_batched(nwc.GemvBatch([b.info for b in blobs], [b.dev for b in blobs], xs, ys, wsp))
    torch.cuda.synchronize()
    assert _counters_zero(blobs, wsp)
    for w, x, y in zip(ws, xs, ys):
        y_ref, a_ref = oracle.gemv(w, x.cpu().numpy())
        _check_y(_to_f64(y), y_ref, a_ref, True, str(w.shape))


# ------------------------------------------------------------ skinny GEMM --

def _gemm(blob: Blob, X: np.ndarray, out_f32: bool):
    Xd = dev(X)
    Y = torch.empty((X.shape[0], blob.info.rows), dtype=torch.float32 if out_f32 else torch.bfloat16,
                    device="cuda")
    nwc.nwc_gemm_skinny(blob.info, blob.dev, Xd, Y, blob.ws(X.shape[0]))
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("batch", [2, 3, 4, 5, 8, 13, 16])
@pytest.mark.parametrize("name,params", [("cfg1", None), ("127x1001", None), ("1000x256", None),
                                         ("cfg1", dict(tile_rows=16)), ("1000x256", dict(tile_rows=16)),
                                         ("cfg1", dict(tile_rows=32)), ("wide_odd", None),
                                         ("cfg1", dict(max_code_len=6)), ("1000x256", dict(tile_rows=16, max_code_len=6))])
def test_gemm_small(name, params, batch):
    w = _special(name)
    X = workloads.gaussian_bits((batch, w.shape[1]), 1.0, 12)
    _say("gemm %s %s batch %d %s" % (name, w.shape, batch, params))
    b = Blob(w, params)
    Y_ref, A_ref = oracle.gemm(w, X)
    for out_f32 in (False, True):
        Y = _to_f64(_gemm(b, X, out_f32))
        for beta in range(batch):
            _check_y(Y[beta], Y_ref[beta], A_ref[beta], out_f32, "%s b%d" % (name, beta))


@pytest.mark.parametrize("rows,cols", [(1003, 4104), (37, 2056), (3000, 512), (4096, 1536), (30000, 1024)])
@pytest.mark.parametrize("batch", [5, 10, 16, 17, 24, 32])
def test_gemm_matrix_core_shapes(rows, cols, batch):
    # the matrix-core skinny GEMM (8-row tiles, batch 5..32: one or two
    # groups of 16 X rows, the second partial at 17 and 24) on shapes whose
    # ranges cut the column groups unevenly: a last column tile of 8 columns
    # (4104), fewer column tiles than matrix-core wavefronts (512, 1536), a
    # last row block of 3 or 5 rows, and ranges of 15 row blocks whose sums
    # are chained column by column (30000 rows); every output within the
    # bound, repeats bitwise equal
    w = workloads.gaussian_bits((rows, cols), 0.02, 71)
    X = workloads.gaussian_bits((batch, cols), 1.0, 72)
    _say("matrix-core gemm %dx%d batch %d" % (rows, cols, batch))
    b = Blob(w)
    Y_ref, A_ref = oracle.gemm(w, X)
    Y = _gemm(b, X, True)
    Y2 = _gemm(b, X, True)
    assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32))
    Yd = _to_f64(Y)
    for beta in range(batch):
        _check_y(Yd[beta], Y_ref[beta], A_ref[beta], True, "%dx%d b%d" % (rows, cols, beta))


def test_gemm_matrix_core_wait_limit_gives_nan_not_a_hang():
    # a one-poll bound makes the matrix-core wavefronts' first waits give up
    # (the decoders take microseconds per tile): the kernel still ends, its
    # outputs are NaN, and with the default bound restored the same call is
    # correct again
    w = workloads.gaussian_bits((4096, 1536), 0.02, 81)
    X = workloads.gaussian_bits((16, 1536), 1.0, 82)
    b = Blob(w)
    _say("wait limit 1")
    try:
        nwc.nwc_set_wait_limit(1)
        Y = _gemm(b, X, True)
    finally:
        nwc.nwc_set_wait_limit(0)
    assert torch.isnan(Y).any()
    Y_ref, A_ref = oracle.gemm(w, X)
    Yd = _to_f64(_gemm(b, X, True))
    for beta in range(16):
        _check_y(Yd[beta], Y_ref[beta], A_ref[beta], True, "restored b%d" % beta)


def test_gemm_deterministic():
    w = _w(4, "w_4096x14336")
    X = workloads.activations(4, "w_4096x14336", batch=16)
    b = Blob(w)
    a = _gemm(b, X, True).cpu().numpy()
    c = _gemm(b, X, True).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))


# ----------------------------------------------------------- row gather ----

@pytest.mark.parametrize("name,params", [("cfg1", None), ("127x1001", None), ("all_patterns", None),
                                         ("cfg1", dict(tile_rows=16)), ("1000x256", dict(tile_rows=32)),
                                         ("cfg1", dict(max_code_len=12)), ("1x1", None),
                                         ("wide_odd", dict(tile_rows=3, tile_cols=7, chunks_per_tile=7,
                                                           max_code_len=10))])
def test_gather_rows_bit_exact(name, params):
    # rows by index, the first and last among them, repeats, and ids past
    # the matrix (a row of zeros)
    w = _special(name)
    rng = np.random.default_rng(21)
    ids = np.concatenate([[0, w.shape[0] - 1], rng.integers(0, w.shape[0], 40), [w.shape[0] // 2] * 3,
                          [w.shape[0], 2 ** 32 - 1]]).astype(np.uint32)
    _say("gather %s %s %s" % (name, w.shape, params))
    b = Blob(w, params)
    ld = -(-w.shape[1] // 8) * 8 + 8
    out = torch.full((len(ids), ld), 0x7E7E, dtype=torch.int16, device="cuda")
    nwc.nwc_gather_rows(b.info, b.dev, dev(ids.view(np.int32)), out[:, :w.shape[1]])
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    want = np.zeros((len(ids), w.shape[1]), np.uint16)
    ok = ids < w.shape[0]
    want[ok] = w[ids[ok]]
    assert np.array_equal(got[:, :w.shape[1]], want)
    assert np.all(got[:, w.shape[1]:] == 0x7E7E)  # nothing written past a row


def test_gather_rows_lm_head():
    # the tied LM head's compressed matrix as the embedding table: 16 tokens
    w = _w(5, "lm_head")
    ids = np.random.default_rng(3).integers(0, w.shape[0], 16).astype(np.uint32)
    b = Blob(w)
    out = torch.empty((16, w.shape[1]), dtype=torch.int16, device="cuda")
    _say("gather lm_head 16 rows")
    nwc.nwc_gather_rows(b.info, b.dev, dev(ids.view(np.int32)), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), w[ids])


# ------------------------------------------- prefill: decode + hipBLASLt ----

_BLAS = []


def _blas():
    if not _BLAS:
        _BLAS.append(nwc.Blas())
    return _BLAS[0]


def _padded(a: np.ndarray, cols_to: int):
    """A device copy of a [rows, cols] array whose rows are cols_to elements apart."""
    out = torch.zeros((a.shape[0], cols_to), dtype=torch.int16, device="cuda")
    out[:, :a.shape[1]] = dev(a.view(np.int16))
    return out[:, :a.shape[1]]


def _prefill(blob: Blob, X: np.ndarray, out_f32: bool):
    up8 = lambda v: -(-v // 8) * 8
    Xd = _padded(X, up8(X.shape[1]))
    Yfull = torch.full((X.shape[0], up8(blob.info.rows)), float("nan"),
                       dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    Y = Yfull[:, :blob.info.rows]
    ws = torch.empty(nwc.nwc_prefill_workspace_size(blob.info), dtype=torch.uint8, device="cuda")
    nwc.nwc_gemm_prefill(_blas(), blob.info, blob.dev, Xd, Y, ws)
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("name,params,batch", [("cfg1", None, 17), ("cfg1", None, 64), ("127x1001", None, 20),
                                               ("1000x256", dict(tile_rows=16), 33), ("wide_odd", None, 40),
                                               ("1x1", None, 17), ("cfg1", dict(max_code_len=12), 100)])
def test_gemm_prefill_small(name, params, batch):
    w = _special(name)
    X = workloads.gaussian_bits((batch, w.shape[1]), 1.0, 14)
    _say("prefill %s %s batch %d %s" % (name, w.shape, batch, params))
    b = Blob(w, params)
    Y_ref, A_ref = oracle.gemm(w, X)
    for out_f32 in (False, True):
        Y = _to_f64(_prefill(b, X, out_f32))
        for beta in range(batch):
            _check_y(Y[beta], Y_ref[beta], A_ref[beta], out_f32, "%s b%d" % (name, beta))


def _sample_rows(n, k=512, seed=0):
    rng = np.random.default_rng(seed)
    idx = np.unique(np.concatenate([rng.choice(n, min(k, n), replace=False), [0, n - 1]]))
    return idx


@pytest.mark.parametrize("name", ["w_4096x14336", "w_14336x4096"])
def test_gemm_prefill_workload_sampled(name):
    w = _w(4, name)
    X = workloads.activations(4, name, batch=64)
    _say("prefill workload 4 %s batch 64" % name)
    b = Blob(w)
    Y = _to_f64(_prefill(b, X, False))
    idx = _sample_rows(w.shape[0], 256, seed=64)
    Y_ref, A_ref = oracle.gemm(np.ascontiguousarray(w[idx]), X)
    for beta in range(0, 64, 7):
        _check_y(Y[beta][idx], Y_ref[beta], A_ref[beta], False, "%s b%d" % (name, beta))


# ------------------------------------------------------- torch module ----

@pytest.mark.parametrize("shape,bias", [((256, 512), True), ((1000, 256), False), ((37, 104), True)])
def test_nwclinear_matches_dense_layer(shape, bias):
    from decode_gemv_byte_amd.linear import NWCLinear
    out_f, in_f = shape
    torch.manual_seed(0)
    lin = torch.nn.Linear(in_f, out_f, bias=bias).to(torch.bfloat16)
    m = NWCLinear.from_linear(lin)
    w = lin.weight.detach().view(torch.int16).numpy().view(np.uint16)
    assert torch.equal(m.dense_weight().cpu().view(torch.int16), lin.weight.detach().view(torch.int16))
    for batch in (1, 3, 16, 40):
        _say("NWCLinear %s batch %d" % (shape, batch))
        x = workloads.gaussian_bits((batch, in_f), 1.0, 30 + batch)
        y = m(torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16).reshape(batch, 1, in_f))
        assert y.shape == (batch, 1, out_f) and y.dtype == torch.bfloat16
        p_ref, a_ref = oracle.gemm(w, x)
        got = _to_f64(y.reshape(batch, out_f))
        y_ref = p_ref
        if bias:
            # the bias is added to the BF16-rounded product: besides the
            # output rounding, one more rounding of 2^-8 |W x| (passed as
            # 4 |W x| in the 2^-10 term)
            y_ref = p_ref + lin.bias.detach().float().numpy().astype(np.float64)
            a_ref = a_ref + 4.0 * np.abs(p_ref)
        for beta in range(batch):
            _check_y(got[beta], y_ref[beta], a_ref[beta], False, "%s b%d" % (shape, beta))


def test_convert_replaces_every_linear():
    # a two-layer net converted in place: each converted layer's output
    # against the oracle's FP64 product of the same BF16 weights and inputs
    # (bound 2^-10 sum|w x| plus one BF16 rounding of the product and, with a
    # bias, one more of the torch bias add), and the net's own forward equal
    # to the layers run one by one
    from decode_gemv_byte_amd.linear import NWCLinear, convert
    torch.manual_seed(1)
    net = torch.nn.Sequential(torch.nn.Linear(512, 256), torch.nn.SiLU(),
                              torch.nn.Sequential(torch.nn.Linear(256, 128, bias=False))).to(torch.bfloat16)
    x = torch.randn(5, 512).to(torch.bfloat16)
    bits = lambda t: t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    w1, b1, w2 = bits(net[0].weight), net[0].bias.detach().double().numpy(), bits(net[2][0].weight)
    convert(net)
    assert isinstance(net[0], NWCLinear) and isinstance(net[2][0], NWCLinear)
    _say("convert: 2-layer net")
    xd = x.cuda()
    y1 = net[0](xd)
    Y1, A1 = oracle.gemm(w1, bits(x))
    got1 = _to_f64(y1)
    for beta in range(5):
        tol = 2.0 ** -10 * A1[beta] + 2.0 ** -8 * np.abs(Y1[beta]) + 2.0 ** -7 * np.abs(Y1[beta] + b1)
        assert np.all(np.abs(got1[beta] - (Y1[beta] + b1)) <= tol), beta
    h1 = net[1](y1)
    y2 = net[2][0](h1)
    Y2, A2 = oracle.gemm(w2, bits(h1))
    got2 = _to_f64(y2)
    for beta in range(5):
        _check_y(got2[beta], Y2[beta], A2[beta], False, "layer 2 row %d" % beta)
    assert torch.equal(net(xd).view(torch.int16), y2.view(torch.int16))


# ------------------------------------------------------ BF16 comparator ----

BF16_CASES = [(1, "w"), (2, "q"), (2, "down"), (3, "gate"), (3, "down"), (3, "k"),
              ("127x1000", None), ("8x512", None), ("20x40960", None)]


@pytest.mark.parametrize("cid,name", BF16_CASES)
def test_gemv_bf16_comparator(cid, name):
    # the comparator runs the fused kernel's pipeline on plain BF16 rows: every
    # row within the bound, the workspace left zero, repeats bitwise equal
    if name is None:
        r, c = (int(v) for v in cid.split("x"))
        w = workloads.gaussian_bits((r, c), 0.02, 61)
        x = workloads.gaussian_bits((c,), 1.0, 62)
    else:
        w = _w(cid, name)
        x = workloads.activations(cid, name)[0]
    _say("bf16 comparator %s %s %s" % (cid, name, w.shape))
    wd = dev(w)
    xd = dev(x)
    ws = torch.zeros(nwc.nwc_bf16_workspace_size(*w.shape), dtype=torch.uint8, device="cuda")
    y_ref, a_ref = oracle.gemv(w, x)
    for out_f32 in (True, False):
        y = torch.empty(w.shape[0], dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
        nwc.nwc_gemv_bf16(wd, xd, y, ws)
        torch.cuda.synchronize()
        _check_y(_to_f64(y), y_ref, a_ref, out_f32, "%s %s" % (cid, name))
        y2 = torch.empty_like(y)
        nwc.nwc_gemv_bf16(wd, xd, y2, ws)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16) if not out_f32 else y.view(torch.int32),
                           y2.view(torch.int16) if not out_f32 else y2.view(torch.int32))
    assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("n16,groups,at", [(1000, 3, 999), (1000, 3, 0), (4099, 7, 2050), (64, 8, 63),
                                           (1 << 20, 0, (1 << 20) - 1)])
def test_read_probe_reads_every_word(layout, n16, groups, at):
    # one 16-byte word whose four dwords XOR to the probe's marker, zeros
    # elsewhere: the lane that loads it (and only that lane) stores the
    # marker, so the sink shows the word was read, at the edges of the
    # workgroups' ranges and the ragged tail too
    _say("read probe layout %d n16 %d groups %d at %d" % (layout, n16, groups, at))
    buf = torch.zeros(n16 * 4, dtype=torch.int32, device="cuda")
    buf[at * 4] = int(np.int32(np.uint32(0x9E3779B9).view(np.int32)))
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    nwc.nwc_read_probe(buf, sink, groups, layout)
    torch.cuda.synchronize()
    assert int(sink.view(torch.int32).item()) == int(np.uint32(0x9E3779B9).view(np.int32))
    sink.zero_()
    buf.zero_()
    nwc.nwc_read_probe(buf, sink, groups, layout)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_native_library_is_in_tree():
    assert os.path.dirname(os.path.abspath(nwc.LIB_PATH)).startswith(ROOT)
    maps = open("/proc/self/maps").read()
    assert nwc.LIB_PATH in maps


def test_gemv_batched_short_codes_and_mixed_limits():
    # all blobs at L = 6 take the second-lookup-free kernel; one blob at L = 8
    # among them sends the whole launch through the general one
    ws = [workloads.gaussian_bits((1000, 256), 0.02, 31), workloads.gaussian_bits((37, 1024), 0.05, 32),
          workloads.gaussian_bits((300, 2048), 0.01, 33)]
    xs = [dev(workloads.gaussian_bits((w.shape[1],), 1.0, 40 + i)) for i, w in enumerate(ws)]
    for limits in ((6, 6, 6), (6, 8, 6)):
        blobs = [Blob(w, dict(max_code_len=l)) for w, l in zip(ws, limits)]
        ys = [torch.empty(w.shape[0], dtype=torch.float32, device="cuda") for w in ws]
        wsp = _batched_ws(blobs)
        _say("gemv_batched limits %s" % (limits,))
        nwc.nwc_gemv_batched(nwc.GemvBatch([b.info for b in blobs], [b.dev for b in blobs], xs, ys, wsp))
        torch.cuda.synchronize()
        assert _counters_zero(blobs, wsp)
        for b, x, y in zip(blobs, xs, ys):
            y_ref, a_ref = oracle.gemv(b.w, x.cpu().numpy())
            _check_y(_to_f64(y), y_ref, a_ref, True, "limits %s" % (limits,))
        outs = [torch.empty(w.shape, dtype=torch.int16, device="cuda") for w in ws]
        nwc.nwc_decode_batched(nwc.DecodeBatch([b.info for b in blobs], [b.dev for b in blobs], outs))
        torch.cuda.synchronize()
        for w, o in zip(ws, outs):
            assert np.array_equal(o.cpu().numpy().view(np.uint16), w)


# ------------------------------------------------------- seeded shape sweep --

def _sweep_cases(n=24, seed=2026):
    # rows, cols, tile rows, code limit, batch: ragged edges in both
    # dimensions, every fast tile height and limits 6 / 8 / 12
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        rows = int(rng.integers(1, 3000))
        cols = int(rng.choice([int(rng.integers(1, 5000)), 8 * int(rng.integers(1, 640))]))
        tr = int(rng.choice([4, 8, 16, 32]))
        lmax = int(rng.choice([6, 8, 12]))
        batch = int(rng.integers(2, 17))
        out.append((i, rows, cols, tr, lmax, batch))
    return out


@pytest.mark.parametrize("i,rows,cols,tr,lmax,batch", _sweep_cases())
def test_seeded_shape_sweep(i, rows, cols, tr, lmax, batch):
    w = workloads.gaussian_bits((rows, cols), float(np.exp(-4 + i % 3)), 500 + i)
    _say("sweep %d: %dx%d TR %d L %d batch %d" % (i, rows, cols, tr, lmax, batch))
    b = Blob(w, dict(tile_rows=tr, max_code_len=lmax))
    out = torch.full(w.shape, 0x5A5A, dtype=torch.int16, device="cuda")
    nwc.nwc_decode(b.info, b.dev, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), w)
    x = workloads.gaussian_bits((cols,), 1.0, 900 + i)
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    nwc.nwc_gemv(b.info, b.dev, dev(x), y, b.ws(1))
    torch.cuda.synchronize()
    y_ref, a_ref = oracle.gemv(w, x)
    _check_y(_to_f64(y), y_ref, a_ref, True, "sweep %d gemv" % i)
    X = workloads.gaussian_bits((batch, cols), 1.0, 1300 + i)
    Y = _to_f64(_gemm(b, X, False))
    Y_ref, A_ref = oracle.gemm(w, X)
    for beta in range(batch):
        _check_y(Y[beta], Y_ref[beta], A_ref[beta], False, "sweep %d b%d" % (i, beta))


@pytest.mark.parametrize("name,params", [("cfg1", dict(pair_fit=1024)), ("3000x512", dict(pair_fit=64)),
                                         ("20x40960", dict(tile_rows=4, pair_fit=1024)),
                                         ("1000x256", dict(tile_rows=16, pair_fit=256))])
def test_pair_fit_blobs_decode_and_multiply(name, params):
    # codes capped at 6 bits for the common exponents: same decoders, exact
    w = _special(name)
    _say("pair_fit %s %s" % (name, params))
    b = Blob(w, params)
    assert np.array_equal(b.host, oracle.encode(w, params.get("tile_rows", 8), 512, 64, 8, params["pair_fit"]))
    out = torch.full(w.shape, 0x5A5A, dtype=torch.int16, device="cuda")
    nwc.nwc_decode(b.info, b.dev, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), w)
    x = workloads.gaussian_bits((w.shape[1],), 1.0, 77)
    y = torch.empty(w.shape[0], dtype=torch.float32, device="cuda")
    nwc.nwc_gemv(b.info, b.dev, dev(x), y, b.ws(1))
    torch.cuda.synchronize()
    y_ref, a_ref = oracle.gemv(w, x)
    _check_y(_to_f64(y), y_ref, a_ref, True, "pair_fit gemv")
    for batch in (4, 8, 16):
        X = workloads.gaussian_bits((batch, w.shape[1]), 1.0, 80 + batch)
        Y = _to_f64(_gemm(b, X, True))
        Y_ref, A_ref = oracle.gemm(w, X)
        for beta in range(batch):
            _check_y(Y[beta], Y_ref[beta], A_ref[beta], True, "pair_fit b%d" % beta)
