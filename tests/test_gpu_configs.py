"""GPU parity on the full-size workloads, in the launches the benchmark times.

For each of the five workloads (seeded synthetic weights from ``workloads``):
* every matrix decodes bit-exactly on the GPU (single and batched decode);
* every output row of the fused products matches the CPU oracle's FP64
  product within 2^-10 * sum|w x| (FP32 output; plus 2^-8 |y| for BF16
  output): batch 1 through the grouped launches of a decode step (q+k+v and
  gate+up in one launch each, o and down alone), batches 2..32 through the
  skinny GEMM, the LM head at batch 1 and 8;
* one-hot inputs make the FP32 output a column of W exactly (each product is
  w * 1 and every other term is a zero), so a single wrongly decoded weight
  in that column shows, which the tolerance above cannot see.  The columns
  cover every position of a lane's 8 columns, the first, a middle and the
  last column tile, and the columns holding the exponents with the longest
  codes (the rare ones, decoded by the second table lookup).

Weights are generated on the host once per module (``functools.lru_cache``);
the oracle's FP64 products of the larger matrices run on a thread pool over
row blocks (its C calls release the interpreter lock).
"""
import functools
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
import decode_gemv_byte_amd as nwc  # noqa: E402

pytestmark = pytest.mark.gpu

LAYER_NAMES = ("q", "k", "v", "o", "gate", "up", "down")
STEP_GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


def _say(msg):
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _threads():
    n = len(os.sched_getaffinity(0))
    try:
        n = min(n, int(os.environ["OMP_NUM_THREADS"]))
    except (KeyError, ValueError):
        pass
    return max(1, min(n, 16))


@functools.lru_cache(maxsize=None)
def _w(cid, name, layer=0):
    return workloads.weights(cid, name, layer=layer)


@functools.lru_cache(maxsize=None)
def _blob(cid, name, layer=0):
    w = _w(cid, name, layer)
    host = nwc.nwc_encode(w)
    return host, nwc.nwc_inspect(host)


def _dev_blob(cid, name, layer=0):
    host, info = _blob(cid, name, layer)
    return info, dev(host)


def _oracle_gemm(w: np.ndarray, X: np.ndarray):
    """FP64 Y = X W^T and A = |X| |W|^T, [batch, rows], over row blocks in parallel."""
    rows = w.shape[0]
    n = _threads()
    cuts = [rows * i // n for i in range(n + 1)]

    def part(i):
        return oracle.gemm(np.ascontiguousarray(w[cuts[i]:cuts[i + 1]]), X)

    with ThreadPoolExecutor(max_workers=n) as ex:
        parts = list(ex.map(part, range(n)))
    return np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts], axis=1)


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
    return t.float().cpu().numpy().astype(np.float64)


def _bf16_as_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _exact_column(y: np.ndarray, col_bits: np.ndarray, what: str):
    """FP32 output of a one-hot product equals the BF16 column exactly (a
    zero weight may come out as +0 or -0: the sum of signed zeros)."""
    want = _bf16_as_f32(col_bits)
    got = np.asarray(y, np.float32)
    bad = np.flatnonzero(~((got == want) & ((got.view(np.uint32) == want.view(np.uint32)) | (want == 0))))
    assert bad.size == 0, "%s: %d wrong weights, first rows %s: got %r want %r" % (
        what, bad.size, bad[:5], got[bad[:5]], want[bad[:5]])


def _probe_columns(w: np.ndarray, info) -> list:
    """Columns whose one-hot product checks the decode: every position of a
    lane's 8 columns (at several lanes) in the first, a middle and the last
    column tile, the last column, and the columns that hold the exponents
    with the longest codes."""
    K = w.shape[1]
    tc = 512
    n_tc = -(-K // tc)
    cols = set()
    for tj in sorted({0, n_tc // 2, n_tc - 1}):
        for j in range(8):
            lane = (7 * j + 3 * tj) % 64
            cols.add(min(K - 1, tj * tc + 8 * lane + j))
    cols.add(K - 1)
    e = (w >> np.uint16(7)) & np.uint16(0xFF)
    lens = np.asarray(info.code_len, np.uint8)
    el = lens[e]
    longest = np.argsort(el.max(axis=0), kind="stable")[::-1][:8]
    cols.update(int(c) for c in longest)
    return sorted(cols)


def _one_hot(K: int, k: int) -> np.ndarray:
    x = np.zeros(K, np.uint16)
    x[k] = 0x3F80     # 1.0
    return x


# ----------------------------------------------- Llama-3.1-8B-shaped step --

@pytest.mark.parametrize("layer", [0, 31])
def test_llama_step_decode_every_matrix(layer):
    # the step's seven matrices: one batched decode launch, and each alone
    infos, blobs, outs = [], [], []
    for n in LAYER_NAMES:
        info, b = _dev_blob(3, n, layer)
        infos.append(info)
        blobs.append(b)
        outs.append(torch.full((info.rows, info.cols), 0x5A5A, dtype=torch.int16, device="cuda"))
    _say("workload 3 layer %d: nwc_decode_batched, 7 matrices" % layer)
    nwc.nwc_decode_batched(nwc.DecodeBatch(infos, blobs, outs))
    torch.cuda.synchronize()
    for n, o in zip(LAYER_NAMES, outs):
        assert torch.equal(o, dev(_w(3, n, layer).view(np.int16))), n
    for n, info, b in zip(LAYER_NAMES, infos, blobs):
        _say("workload 3 layer %d: nwc_decode %s" % (layer, n))
        o = torch.full((info.rows, info.cols), 0x5A5A, dtype=torch.int16, device="cuda")
        nwc.nwc_decode(info, b, o)
        torch.cuda.synchronize()
        assert torch.equal(o, dev(_w(3, n, layer).view(np.int16))), n


@functools.lru_cache(maxsize=None)
def _llama_ref(layer, name):
    Y, A = _oracle_gemm(_w(3, name, layer), workloads.activations(3, name, layer=layer))
    return Y[0], A[0]


@pytest.mark.parametrize("out_f32", [False, True])
@pytest.mark.parametrize("layer", [0, 31])
def test_llama_step_gemv_all_rows(layer, out_f32):
    # the launches bench.py times for a decode step, every row of every matrix
    dt = torch.float32 if out_f32 else torch.bfloat16
    for grp in STEP_GROUPS:
        infos, blobs, xs, ys = [], [], [], []
        for n in grp:
            info, b = _dev_blob(3, n, layer)
            infos.append(info)
            blobs.append(b)
            xs.append(workloads.activations(3, n, layer=layer)[0])
            ys.append(torch.empty(info.rows, dtype=dt, device="cuda"))
        _say("workload 3 layer %d: %s f32=%s" % (layer, "+".join(grp), out_f32))
        if len(grp) > 1:
            ws = torch.zeros(nwc.gemv_batched_workspace_size(infos), dtype=torch.uint8, device="cuda")
            nwc.nwc_gemv_batched(nwc.GemvBatch(infos, blobs, [dev(x) for x in xs], ys, ws))
        else:
            ws = torch.zeros(nwc.nwc_workspace_size(infos[0], 1), dtype=torch.uint8, device="cuda")
            nwc.nwc_gemv(infos[0], blobs[0], dev(xs[0]), ys[0], ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0
        for n, y in zip(grp, ys):
            Y, A = _llama_ref(layer, n)
            _check_y(_to_f64(y), Y, A, out_f32, "layer %d %s" % (layer, n))


@pytest.mark.parametrize("layer", [0, 31])
def test_llama_step_one_hot_columns_exact(layer):
    # one-hot x through the same launches: y is column k of W, bit for bit
    for grp in STEP_GROUPS:
        infos, blobs = zip(*[_dev_blob(3, n, layer) for n in grp])
        K = infos[0].cols
        cols = sorted(set().union(*[_probe_columns(_w(3, n, layer), i) for n, i in zip(grp, infos)]))
        _say("workload 3 layer %d: one-hot %s, %d columns" % (layer, "+".join(grp), len(cols)))
        ys = [torch.empty(i.rows, dtype=torch.float32, device="cuda") for i in infos]
        ws = torch.zeros(nwc.gemv_batched_workspace_size(list(infos)), dtype=torch.uint8, device="cuda")
        for k in cols:
            xd = dev(_one_hot(K, k))
            if len(grp) > 1:
                nwc.nwc_gemv_batched(nwc.GemvBatch(list(infos), list(blobs), [xd] * len(grp), ys, ws))
            else:
                nwc.nwc_gemv(infos[0], blobs[0], xd, ys[0], ws)
            torch.cuda.synchronize()
            for n, y in zip(grp, ys):
                _exact_column(y.cpu().numpy(), _w(3, n, layer)[:, k], "layer %d %s column %d" % (layer, n, k))


# ------------------------------------------------------ skinny decode-GEMM --

@pytest.mark.parametrize("name", ["w_4096x14336", "w_14336x4096"])
def test_skinny_decode_bit_exact(name):
    info, b = _dev_blob(4, name)
    out = torch.full((info.rows, info.cols), 0x5A5A, dtype=torch.int16, device="cuda")
    _say("workload 4 decode %s" % name)
    nwc.nwc_decode(info, b, out)
    torch.cuda.synchronize()
    assert torch.equal(out, dev(_w(4, name).view(np.int16)))


@functools.lru_cache(maxsize=None)
@functools.lru_cache(maxsize=None)
def _skinny_ref(name):
    # the batch rows of every batch size are the first rows of the same draw
    X = workloads.activations(4, name, batch=32)
    return X, _oracle_gemm(_w(4, name), X)


@pytest.mark.parametrize("batch", [2, 3, 4, 8, 9, 12, 16, 32])
@pytest.mark.parametrize("name", ["w_4096x14336", "w_14336x4096"])
def test_skinny_gemm_all_rows(name, batch):
    info, b = _dev_blob(4, name)
    X32, (Y16, A16) = _skinny_ref(name)
    X = X32[:batch]
    assert np.array_equal(X, workloads.activations(4, name, batch=batch))
    ws = torch.zeros(max(1, nwc.nwc_workspace_size(info, batch)), dtype=torch.uint8, device="cuda")
    for out_f32 in (False, True):
        _say("workload 4 %s batch %d f32=%s" % (name, batch, out_f32))
        Y = torch.empty((batch, info.rows), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
        nwc.nwc_gemm_skinny(info, b, dev(X), Y, ws)
        torch.cuda.synchronize()
        Yh = _to_f64(Y)
        for beta in range(batch):
            _check_y(Yh[beta], Y16[beta], A16[beta], out_f32, "%s batch %d row %d" % (name, batch, beta))


@pytest.mark.parametrize("batch", [2, 4, 8, 16])
@pytest.mark.parametrize("name", ["w_4096x14336", "w_14336x4096"])
def test_skinny_one_hot_columns_exact(name, batch):
    # X row beta one-hot at its own column: Y row beta is that column of W
    info, b = _dev_blob(4, name)
    w = _w(4, name)
    cols = _probe_columns(w, info)
    ws = torch.zeros(max(1, nwc.nwc_workspace_size(info, batch)), dtype=torch.uint8, device="cuda")
    _say("workload 4 %s batch %d one-hot, %d columns" % (name, batch, len(cols)))
    for c0 in range(0, len(cols), batch):
        ks = [cols[(c0 + i) % len(cols)] for i in range(batch)]
        X = np.stack([_one_hot(info.cols, k) for k in ks])
        Y = torch.empty((batch, info.rows), dtype=torch.float32, device="cuda")
        nwc.nwc_gemm_skinny(info, b, dev(X), Y, ws)
        torch.cuda.synchronize()
        Yh = Y.cpu().numpy()
        for beta, k in enumerate(ks):
            _exact_column(Yh[beta], w[:, k], "%s batch %d row %d column %d" % (name, batch, beta, k))


# --------------------------------------------------------------- LM head --

def test_lm_head_decode_bit_exact():
    info, b = _dev_blob(5, "lm_head")
    out = torch.empty((info.rows, info.cols), dtype=torch.int16, device="cuda")
    _say("workload 5 decode lm_head")
    nwc.nwc_decode(info, b, out)
    torch.cuda.synchronize()
    assert torch.equal(out, dev(_w(5, "lm_head").view(np.int16)))


@functools.lru_cache(maxsize=None)
def _lm_ref():
    X = workloads.activations(5, "lm_head", batch=8)
    return X, _oracle_gemm(_w(5, "lm_head"), X)


def test_lm_head_gemv_all_rows():
    info, b = _dev_blob(5, "lm_head")
    X8, (Y8, A8) = _lm_ref()
    x = workloads.activations(5, "lm_head", batch=1)[0]
    assert np.array_equal(x, X8[0])
    ws = torch.zeros(nwc.nwc_workspace_size(info, 1), dtype=torch.uint8, device="cuda")
    for out_f32 in (False, True):
        _say("workload 5 lm_head batch 1 f32=%s" % out_f32)
        y = torch.empty(info.rows, dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
        nwc.nwc_gemv(info, b, dev(x), y, ws)
        torch.cuda.synchronize()
        _check_y(_to_f64(y), Y8[0], A8[0], out_f32, "lm_head batch 1")
    assert int(ws.count_nonzero()) == 0


def test_lm_head_batch8_all_rows():
    info, b = _dev_blob(5, "lm_head")
    X8, (Y8, A8) = _lm_ref()
    ws = torch.zeros(max(1, nwc.nwc_workspace_size(info, 8)), dtype=torch.uint8, device="cuda")
    for out_f32 in (False, True):
        _say("workload 5 lm_head batch 8 f32=%s" % out_f32)
        Y = torch.empty((8, info.rows), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
        nwc.nwc_gemm_skinny(info, b, dev(X8), Y, ws)
        torch.cuda.synchronize()
        Yh = _to_f64(Y)
        for beta in range(8):
            _check_y(Yh[beta], Y8[beta], A8[beta], out_f32, "lm_head batch 8 row %d" % beta)


def test_lm_head_one_hot_columns_exact():
    info, b = _dev_blob(5, "lm_head")
    w = _w(5, "lm_head")
    cols = _probe_columns(w, info)
    ws = torch.zeros(nwc.nwc_workspace_size(info, 1), dtype=torch.uint8, device="cuda")
    y = torch.empty(info.rows, dtype=torch.float32, device="cuda")
    _say("workload 5 lm_head one-hot, %d columns" % len(cols))
    for k in cols:
        nwc.nwc_gemv(info, b, dev(_one_hot(info.cols, k)), y, ws)
        torch.cuda.synchronize()
        _exact_column(y.cpu().numpy(), w[:, k], "lm_head column %d" % k)


# ------------------------------------------- single matrix and one layer --

def test_single_matrix_one_hot_every_column():
    # the 1024 x 1024 matrix: every column, each one-hot product exact
    w = _w(1, "w")
    info, b = _dev_blob(1, "w")
    ws = torch.zeros(nwc.nwc_workspace_size(info, 1), dtype=torch.uint8, device="cuda")
    ys = torch.empty((w.shape[1], w.shape[0]), dtype=torch.float32, device="cuda")
    _say("workload 1 one-hot, all 1024 columns")
    for k in range(w.shape[1]):
        nwc.nwc_gemv(info, b, dev(_one_hot(w.shape[1], k)), ys[k], ws)
    torch.cuda.synchronize()
    got = ys.cpu().numpy()
    for k in range(w.shape[1]):
        _exact_column(got[k], w[:, k], "column %d" % k)


@pytest.mark.parametrize("params", [dict(max_code_len=6), dict(max_code_len=8), dict(max_code_len=11),
                                    dict(tile_rows=4), dict(tile_rows=16), dict(tile_rows=32),
                                    dict(tile_rows=5, tile_cols=24, chunks_per_tile=3, max_code_len=11),
                                    dict(tile_rows=3, tile_cols=7, chunks_per_tile=7, max_code_len=10)])
def test_one_hot_columns_other_geometries(params):
    # the same exactness through the other code limits and tile heights and
    # the generic kernels (odd geometries), batch 1 and the skinny GEMM, on a
    # ragged matrix with rare exponents (outliers and tiny weights)
    rng = np.random.default_rng(17)
    w = workloads.gaussian_bits((333, 1000), 0.02, 71)
    rare = rng.random(w.shape) < 0.002
    w[rare] = workloads.gaussian_bits((int(rare.sum()),), 2.0, 72)
    tiny = rng.random(w.shape) < 0.002
    w[tiny] = workloads.gaussian_bits((int(tiny.sum()),), 1e-30, 73)
    host = nwc.nwc_encode(w, params)
    info = nwc.nwc_inspect(host)
    b = dev(host)
    cols = _probe_columns(w, info)
    _say("one-hot geometry %s, %d columns" % (params, len(cols)))
    ws1 = torch.zeros(max(1, nwc.nwc_workspace_size(info, 1)), dtype=torch.uint8, device="cuda")
    y = torch.empty(info.rows, dtype=torch.float32, device="cuda")
    for k in cols:
        nwc.nwc_gemv(info, b, dev(_one_hot(info.cols, k)), y, ws1)
        torch.cuda.synchronize()
        _exact_column(y.cpu().numpy(), w[:, k], "%s column %d" % (params, k))
    batch = 16
    wsb = torch.zeros(max(1, nwc.nwc_workspace_size(info, batch)), dtype=torch.uint8, device="cuda")
    for c0 in range(0, len(cols), batch):
        ks = [cols[(c0 + i) % len(cols)] for i in range(batch)]
        Y = torch.empty((batch, info.rows), dtype=torch.float32, device="cuda")
        nwc.nwc_gemm_skinny(info, b, dev(np.stack([_one_hot(info.cols, k) for k in ks])), Y, wsb)
        torch.cuda.synchronize()
        Yh = Y.cpu().numpy()
        for beta, k in enumerate(ks):
            _exact_column(Yh[beta], w[:, k], "%s skinny column %d" % (params, k))


# ------------------------------- the ranked unary code family (escape index) --

@pytest.mark.parametrize("lmax", [9, 12])
def test_unary_family_parity(lmax):
    # blobs of the second code family decode and multiply through the same
    # kernels: decode bit-exact, every GEMV row within the bound, one-hot
    # columns exact (batch 1 and the skinny GEMM)
    w = _w(3, "gate")
    host = nwc.nwc_encode(w, dict(code_family=1, max_code_len=lmax))
    info = nwc.nwc_inspect(host)
    b = dev(host)
    _say("unary family L=%d: decode, GEMV, one-hot" % lmax)
    out = torch.empty((info.rows, info.cols), dtype=torch.int16, device="cuda")
    nwc.nwc_decode(info, b, out)
    torch.cuda.synchronize()
    assert torch.equal(out, dev(w.view(np.int16)))
    ws = torch.zeros(nwc.nwc_workspace_size(info, 1), dtype=torch.uint8, device="cuda")
    y = torch.empty(info.rows, dtype=torch.float32, device="cuda")
    nwc.nwc_gemv(info, b, dev(workloads.activations(3, "gate")[0]), y, ws)
    torch.cuda.synchronize()
    Y, A = _llama_ref(0, "gate")
    _check_y(_to_f64(y), Y, A, True, "unary L=%d" % lmax)
    for k in _probe_columns(w, info)[:12]:
        nwc.nwc_gemv(info, b, dev(_one_hot(info.cols, k)), y, ws)
        torch.cuda.synchronize()
        _exact_column(y.cpu().numpy(), w[:, k], "unary L=%d column %d" % (lmax, k))
    X = np.stack([_one_hot(info.cols, k) for k in range(0, 16 * 211, 211)])
    Ys = torch.empty((16, info.rows), dtype=torch.float32, device="cuda")
    nwc.nwc_gemm_skinny(info, b, dev(X), Ys, torch.zeros(max(1, nwc.nwc_workspace_size(info, 16)),
                                                         dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    Yh = Ys.cpu().numpy()
    for beta, k in enumerate(range(0, 16 * 211, 211)):
        _exact_column(Yh[beta], w[:, k], "unary L=%d skinny column %d" % (lmax, k))
