"""Host side of libnwc on the CPU: exported symbols, encoder byte identity with
the oracle, blob validation, and argument checks that must fail before any
device work."""
import ctypes
import os
import sys
import re
import subprocess

import numpy as np
import pytest

import decode_gemv_byte_amd as nwc
import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nwc.h")

DEFAULT = dict(tile_rows=8, tile_cols=512, chunks_per_tile=64, max_code_len=8, pair_fit=1024)


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nwc_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", nwc.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (nwc_[a-z0-9_]+)$", out, flags=re.M))
    for n in names:
        assert n in exported, n
        assert hasattr(ctypes.CDLL(nwc.LIB_PATH), n)
    assert set(nwc.EXPORTS) == set(names)


def test_status_strings():
    for s in range(0, -7, -1):
        assert nwc.nwc_status_str(s).startswith("NWC_")
    assert nwc.nwc_status_str(-99) == "NWC_ERR_UNKNOWN"


def _oracle_blob(w, p):
    q = dict(DEFAULT)
    q.update(p or {})
    return oracle.encode(w, q["tile_rows"], q["tile_cols"], q["chunks_per_tile"], q["max_code_len"], q["pair_fit"])


GEOMS = [None, dict(tile_rows=16), dict(tile_rows=32), dict(tile_rows=5, tile_cols=24, chunks_per_tile=3,
                                                              max_code_len=11),
         dict(tile_rows=3, tile_cols=7, chunks_per_tile=7, max_code_len=10), dict(max_code_len=12)]


@pytest.mark.parametrize("geom", GEOMS)
@pytest.mark.parametrize("name", ["cfg1", "all_patterns", "127x1001", "subnormal", "one_symbol", "1x1",
                                  "random_bits"])
def test_encoder_bytes_equal_oracle(name, geom):
    rng = np.random.default_rng(5)
    w = {
        "cfg1": lambda: workloads.weights(1, "w"),
        "all_patterns": workloads.all_patterns,
        "127x1001": lambda: workloads.gaussian_bits((127, 1001), 0.02, 4),
        "subnormal": lambda: (rng.integers(1, 128, (48, 70)) | (rng.integers(0, 2, (48, 70)) << 15)).astype(np.uint16),
        "one_symbol": lambda: (0x3C00 | rng.integers(0, 128, (50, 60))).astype(np.uint16),
        "1x1": lambda: workloads.gaussian_bits((1, 1), 0.02, 1),
        "random_bits": lambda: workloads.random_bits((300, 257), 6),
    }[name]()
    assert np.array_equal(nwc.nwc_encode(w, geom), _oracle_blob(w, geom))


@pytest.mark.parametrize("cid,name", [(2, "q"), (2, "down"), (3, "gate"), (4, "w_4096x14336"), (5, "lm_head")])
def test_encoder_bytes_equal_oracle_workload_slices(cid, name):
    w = workloads.weights(cid, name, rows=slice(0, 512))
    assert np.array_equal(nwc.nwc_encode(w), _oracle_blob(w, None))


def test_encoder_strided_input():
    big = workloads.gaussian_bits((40, 300), 0.02, 3)
    view = big[:, 10:250]
    assert not view.flags.c_contiguous
    assert np.array_equal(nwc.nwc_encode(view), _oracle_blob(np.ascontiguousarray(view), None))


def test_inspect_matches_oracle_header():
    w = workloads.weights(1, "w")
    blob = nwc.nwc_encode(w)
    info = nwc.nwc_inspect(blob)
    h = oracle.header(blob)
    for k in ("rows", "cols", "tile_rows", "tile_cols", "chunks_per_tile", "max_code_len", "n_tiles",
              "n_chunks", "raw_ld", "stream_words", "off_code_len", "off_table", "off_tile_words",
              "off_chunk_bits", "off_raw", "off_stream"):
        assert getattr(info, k) == h[k], k
    assert info.blob_bytes == h["total_bytes"] == blob.size
    sec = oracle.sections(blob)
    assert info.max_tile_words == int(np.diff(sec["tile_words"].astype(np.int64)).max())
    assert info.payload_bits == int(sec["chunk_bits"].astype(np.int64).sum())
    assert info.max_chunk_bits == int(sec["chunk_bits"].max())
    assert bytes(info.code_len) == bytes(sec["code_len"])
    e, _ = oracle.split(w)
    assert info.n_symbols == int((oracle.histogram(e) > 0).sum())


def _corrupt(blob):
    h = oracle.header(blob)
    out = {}
    b = blob.copy(); b[0] ^= 1; out["magic"] = b
    b = blob.copy(); b[4] = 9; out["version"] = b
    out["truncated"] = blob[: blob.size - 300].copy()
    b = blob.copy(); b[h["off_table"] + 40] ^= 0x10; out["table"] = b
    b = blob.copy(); b[h["off_tile_words"] + 8] ^= 0x01; out["tile_words"] = b
    b = blob.copy(); b[h["off_chunk_bits"] + 1] ^= 0x40; out["chunk_bits_range"] = b
    b = blob.copy(); lens = b[h["off_code_len"]: h["off_code_len"] + 256]
    nz = np.flatnonzero(lens)
    lens[nz[0]] = 1; lens[nz[1]] = 1; lens[nz[2]] = 1; out["kraft"] = b
    b = blob.copy(); b[h["off_code_len"] + nz[0]] = 13; out["too_long"] = b
    b = blob.copy(); b[8] ^= 0x01; out["rows"] = b
    b = blob.copy(); b[28] = 0x07; out["geometry"] = b
    b = blob.copy(); b[44] = 1; out["flags"] = b
    b = blob.copy(); b[40] = 2; out["table_kind"] = b
    return out


def test_inspect_rejects_corruption():
    w = workloads.gaussian_bits((127, 1001), 0.02, 4)
    blob = nwc.nwc_encode(w)
    for name, bad in _corrupt(blob).items():
        with pytest.raises(nwc.NwcError) as ei:
            nwc.nwc_inspect(bad)
        assert ei.value.status == nwc.NWC_ERR_BAD_FORMAT, name
        assert oracle.validate(bad) != 0, name


def test_encode_errors():
    w = workloads.gaussian_bits((10, 20), 0.02, 1)
    for p in [dict(tile_cols=500), dict(max_code_len=13), dict(max_code_len=5),
              dict(tile_rows=4096, tile_cols=4096, chunks_per_tile=1)]:
        with pytest.raises(nwc.NwcError) as ei:
            nwc.nwc_encode(w, p)
        assert ei.value.status == nwc.NWC_ERR_INVALID_ARG
    # capacity too small reports the needed size
    need = nwc.nwc_encode(w).size
    buf = np.zeros(need - 1, np.uint8)
    used = ctypes.c_size_t(0)
    st = nwc._lib.nwc_encode(w.ctypes.data, 10, 20, 20, None, buf.ctypes.data, buf.size, ctypes.byref(used))
    assert st == nwc.NWC_ERR_BUFFER_TOO_SMALL and used.value == need
    st = nwc._lib.nwc_encode(None, 10, 20, 20, None, buf.ctypes.data, buf.size, ctypes.byref(used))
    assert st == nwc.NWC_ERR_INVALID_ARG
    assert nwc._lib.nwc_encode(w.ctypes.data, 10, 20, 19, None, buf.ctypes.data, buf.size,
                               ctypes.byref(used)) == nwc.NWC_ERR_INVALID_ARG
    assert nwc.nwc_encode_bound(10, 20) >= need
    # limits below 8 hold at most 2^L distinct exponents
    many = workloads.random_bits((64, 64), 3)
    for lmax in (6, 7):
        with pytest.raises(nwc.NwcError) as ei:
            nwc.nwc_encode(many, dict(max_code_len=lmax))
        assert ei.value.status == nwc.NWC_ERR_INVALID_ARG


@pytest.mark.parametrize("geom", [dict(max_code_len=6), dict(max_code_len=7), dict(tile_rows=4, max_code_len=6)])
@pytest.mark.parametrize("name", ["cfg1", "127x1001", "subnormal", "one_symbol", "1x1"])
def test_encoder_bytes_equal_oracle_short_codes(name, geom):
    # tensors with at most 64 distinct exponent values
    rng = np.random.default_rng(6)
    w = {
        "cfg1": lambda: workloads.weights(1, "w"),
        "127x1001": lambda: workloads.gaussian_bits((127, 1001), 0.05, 3),
        "subnormal": lambda: (rng.integers(1, 128, (48, 70)) | (rng.integers(0, 2, (48, 70)) << 15)).astype(np.uint16),
        "one_symbol": lambda: (0x3C00 | rng.integers(0, 128, (50, 60))).astype(np.uint16),
        "1x1": lambda: workloads.gaussian_bits((1, 1), 0.02, 1),
    }[name]()
    blob = nwc.nwc_encode(w, geom)
    assert np.array_equal(blob, _oracle_blob(w, geom))
    assert nwc.nwc_inspect(blob).max_code_len == geom["max_code_len"]


def test_workspace_sizes():
    # generic geometry (cols % 8 != 0): partial sums per column tile
    blob = nwc.nwc_encode(workloads.gaussian_bits((100, 1500), 0.02, 2))
    info = nwc.nwc_inspect(blob)
    assert nwc.nwc_workspace_size(info, 1) == 3 * 100 * 4
    assert nwc.nwc_workspace_size(info, 16) == 3 * 16 * 100 * 4
    assert nwc.nwc_workspace_size(info, 32) == 3 * 32 * 100 * 4
    for bad in (0, 33):
        with pytest.raises(nwc.NwcError):
            nwc.nwc_workspace_size(info, bad)
    # fused batch 1: one 64-bit chain slot per (tile, row), rounded up to 256
    # bytes; the fused skinny path needs none
    up = lambda v: -(-v // 256) * 256
    fast = nwc.nwc_inspect(nwc.nwc_encode(workloads.gaussian_bits((100, 1504), 0.02, 2)))
    assert nwc.nwc_workspace_size(fast, 1) == up(13 * 3 * 8 * 8)
    tr16 = nwc.nwc_inspect(nwc.nwc_encode(workloads.gaussian_bits((100, 1504), 0.02, 2), dict(tile_rows=16)))
    assert nwc.nwc_workspace_size(tr16, 1) == up(7 * 3 * 16 * 8)
    assert nwc.nwc_workspace_size(tr16, 8) == 0
    assert nwc.nwc_workspace_size(fast, 8) == 0
    # up to 32 X rows: 8-row tiles on the matrix cores (no workspace), other
    # tile heights past 16 rows on the generic path
    assert nwc.nwc_workspace_size(fast, 32) == 0
    assert nwc.nwc_workspace_size(tr16, 17) == 3 * 17 * 100 * 4
    assert nwc.gemv_batched_workspace_size([fast, tr16]) == (nwc.nwc_workspace_size(fast, 1) +
                                                             nwc.nwc_workspace_size(tr16, 1))
    # batch > 1 with tile_rows 32 takes the generic path
    tr32 = nwc.nwc_inspect(nwc.nwc_encode(workloads.gaussian_bits((100, 1504), 0.02, 2), dict(tile_rows=32)))
    assert nwc.nwc_workspace_size(tr32, 1) == up(4 * 3 * 32 * 8)
    assert nwc.nwc_workspace_size(tr32, 8) == 3 * 8 * 100 * 4
    # the comparator: one 64-bit exchange slot per 8-row tile row (13 x 3 tiles of 8 x 512)
    assert nwc.nwc_bf16_workspace_size(100, 1500) == up(13 * 3 * 8 * 8)


def test_device_calls_validate_before_launch():
    # Every call below fails on the host before any device work, so it is safe
    # with fake device addresses (never dereferenced) and runs without a GPU.
    # Do not add a call here that passes validation: it would launch a kernel
    # on the fake addresses.
    blob = nwc.nwc_encode(workloads.gaussian_bits((64, 512), 0.02, 2))
    info = nwc.nwc_inspect(blob)
    L = nwc._lib
    ref = ctypes.byref(info)
    A = 0x10000          # 256-aligned fake device address
    W = nwc.nwc_workspace_size(info, 1)
    assert W > 0
    assert L.nwc_gemv(None, A, A, A, 0, A, W, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv(ref, None, A, A, 0, A, W, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv(ref, A, None, A, 0, A, W, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv(ref, A, A, None, 0, A, W, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv(ref, A, A, A, 7, A, W, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv(ref, A + 16, A, A, 0, A, W, None) == nwc.NWC_ERR_ALIGNMENT
    assert L.nwc_gemv(ref, A, A, A + 1, 0, A, W, None) == nwc.NWC_ERR_ALIGNMENT
    assert L.nwc_gemv(ref, A, A + 2, A, 0, A, W, None) == nwc.NWC_ERR_ALIGNMENT   # x must be 16-aligned
    # the fused path's workspace: present, large enough, 256-byte aligned
    assert L.nwc_gemv(ref, A, A, A, 0, None, 0, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv(ref, A, A, A, 0, A, W - 4, None) == nwc.NWC_ERR_BUFFER_TOO_SMALL
    assert L.nwc_gemv(ref, A, A, A, 0, A + 16, W, None) == nwc.NWC_ERR_ALIGNMENT
    for batch in (0, 1, 33):
        assert L.nwc_gemm_skinny(ref, A, A, 512, batch, A, 64, 0, None, 0, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemm_skinny(ref, A, A, 100, 4, A, 64, 0, None, 0, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemm_skinny(ref, A, A, 512, 4, A, 63, 0, None, 0, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_decode(ref, A, None, 512, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_decode(ref, A, A, 100, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_decode(ref, A + 8, A, 512, None) == nwc.NWC_ERR_ALIGNMENT
    assert L.nwc_decode(ref, A, A + 1, 512, None) == nwc.NWC_ERR_ALIGNMENT
    bad = nwc.nwc_info.from_buffer_copy(info)
    bad.n_tiles += 1
    assert L.nwc_gemv(ctypes.byref(bad), A, A, A, 0, A, W, None) == nwc.NWC_ERR_INVALID_ARG
    # the generic path (odd geometry) needs its workspace
    gblob = nwc.nwc_encode(workloads.gaussian_bits((64, 500), 0.02, 2))
    ginfo = nwc.nwc_inspect(gblob)
    gws = nwc.nwc_workspace_size(ginfo, 1)
    assert gws > 0
    gref = ctypes.byref(ginfo)
    assert L.nwc_gemv(gref, A, A, A, 0, None, 0, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv(gref, A, A, A, 0, A, gws - 4, None) == nwc.NWC_ERR_BUFFER_TOO_SMALL
    assert L.nwc_gemv(gref, A, A, A, 0, A + 4, gws, None) == nwc.NWC_ERR_ALIGNMENT
    BW = nwc.nwc_bf16_workspace_size(64, 512)
    assert L.nwc_gemv_bf16(A, 64, 512, 500, A, A, 0, A, BW, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv_bf16(A, 64, 512, 512, A, A, 0, None, BW, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv_bf16(A, 64, 500, 512, A, A, 0, A, BW, None) == nwc.NWC_ERR_ALIGNMENT
    assert L.nwc_gemv_bf16(A, 64, 512, 512, A + 8, A, 0, A, BW, None) == nwc.NWC_ERR_ALIGNMENT
    assert L.nwc_gemv_bf16(A, 64, 512, 512, A, A, 0, A + 16, BW, None) == nwc.NWC_ERR_ALIGNMENT
    assert L.nwc_gemv_bf16(A, 64, 512, 512, A, A, 0, A, BW - 8, None) == nwc.NWC_ERR_BUFFER_TOO_SMALL
    # the read probe
    assert L.nwc_read_probe(None, 1 << 20, A, 0, 1, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_read_probe(A, 8, A, 0, 1, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_read_probe(A, 1 << 20, A, 0, 2, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_read_probe(A, 1 << 20, A, 0, -1, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_read_probe(A + 8, 1 << 20, A, 0, 0, None) == nwc.NWC_ERR_ALIGNMENT
    assert L.nwc_read_probe(A, 1 << 20, A + 2, 0, 1, None) == nwc.NWC_ERR_ALIGNMENT
    # grouped launch: count, NULL arrays, per-entry checks, geometry mix
    infos = (nwc.nwc_info * 2)(info, info)
    V2 = ctypes.c_void_p * 2
    ok = V2(A, A)
    B = 2 * W
    for count in (0, 9):
        assert L.nwc_gemv_batched(count, infos, ok, ok, ok, 0, A, B, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv_batched(2, None, ok, ok, ok, 0, A, B, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv_batched(2, infos, ok, ok, ok, 5, A, B, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv_batched(2, infos, ok, V2(A, None), ok, 0, A, B, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv_batched(2, infos, ok, ok, ok, 0, None, B, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv_batched(2, infos, V2(A, A + 16), ok, ok, 0, A, B, None) == nwc.NWC_ERR_ALIGNMENT
    assert L.nwc_gemv_batched(2, infos, ok, V2(A, A + 4), ok, 0, A, B, None) == nwc.NWC_ERR_ALIGNMENT
    assert L.nwc_gemv_batched(2, infos, ok, ok, ok, 0, A + 16, B, None) == nwc.NWC_ERR_ALIGNMENT
    assert L.nwc_gemv_batched(2, infos, ok, ok, ok, 0, A, B - 4, None) == nwc.NWC_ERR_BUFFER_TOO_SMALL
    mixed = (nwc.nwc_info * 2)(info, nwc.nwc_inspect(nwc.nwc_encode(workloads.gaussian_bits((64, 512), 0.02, 2),
                                                                      dict(tile_rows=16))))
    assert L.nwc_gemv_batched(2, mixed, ok, ok, ok, 0, A, 1 << 20, None) == nwc.NWC_ERR_UNSUPPORTED
    gen = (nwc.nwc_info * 2)(info, ginfo)
    assert L.nwc_gemv_batched(2, gen, ok, ok, ok, 0, A, 1 << 20, None) == nwc.NWC_ERR_UNSUPPORTED
    # grouped decode: count, NULL arrays, row strides, alignment, geometry mix
    U2 = ctypes.c_uint64 * 2
    lds = U2(info.cols, info.cols)
    for count in (0, 9):
        assert L.nwc_decode_batched(count, infos, ok, ok, lds, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_decode_batched(2, None, ok, ok, lds, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_decode_batched(2, infos, ok, ok, None, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_decode_batched(2, infos, ok, V2(A, None), lds, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_decode_batched(2, infos, ok, ok, U2(info.cols, info.cols - 1), None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_decode_batched(2, infos, ok, V2(A, A + 8), lds, None) == nwc.NWC_ERR_ALIGNMENT
    assert L.nwc_decode_batched(2, infos, ok, ok, U2(info.cols, info.cols + 4), None) == nwc.NWC_ERR_ALIGNMENT
    assert L.nwc_decode_batched(2, mixed, ok, ok, U2(info.cols, 512), None) == nwc.NWC_ERR_UNSUPPORTED
    assert L.nwc_decode_batched(2, gen, ok, ok, U2(info.cols, 500), None) == nwc.NWC_ERR_UNSUPPORTED


def test_prefill_validation():
    # everything here fails before any device work, so it runs without a GPU
    L = nwc._lib
    blob = nwc.nwc_encode(workloads.gaussian_bits((100, 1000), 0.02, 2))
    info = nwc.nwc_inspect(blob)
    need = nwc.nwc_prefill_workspace_size(info)
    assert need == -(-100 * 1000 * 2 // 256) * 256 + (32 << 20)
    A = 1 << 20  # a 256-byte aligned stand-in address (never dereferenced)
    h = ctypes.c_void_p(A)
    ok = ctypes.c_void_p(A)
    call = lambda h_, batch=20, ldx=1000, ldy=104, X=ok, Y=ok, ws=ok, n=need, yt=0: L.nwc_gemm_prefill(
        h_, ctypes.byref(info), ok, X, ldx, batch, Y, ldy, yt, ws, n, None)
    assert call(None) == nwc.NWC_ERR_INVALID_ARG
    assert call(h, batch=0) == nwc.NWC_ERR_INVALID_ARG
    assert call(h, ldx=999) == nwc.NWC_ERR_INVALID_ARG
    assert call(h, ldy=99) == nwc.NWC_ERR_INVALID_ARG
    assert call(h, yt=7) == nwc.NWC_ERR_INVALID_ARG
    assert call(h, X=None) == nwc.NWC_ERR_INVALID_ARG
    assert call(h, n=need - 1) == nwc.NWC_ERR_BUFFER_TOO_SMALL
    assert call(h, X=ctypes.c_void_p(A + 2)) == nwc.NWC_ERR_ALIGNMENT
    assert call(h, ws=ctypes.c_void_p(A + 16)) == nwc.NWC_ERR_ALIGNMENT
    assert call(h, ldx=1004) == nwc.NWC_ERR_ALIGNMENT
    assert call(h, ldy=100) == nwc.NWC_ERR_ALIGNMENT
    assert L.nwc_blas_create(None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_blas_destroy(None) == nwc.NWC_ERR_INVALID_ARG
    with pytest.raises(nwc.NwcError):
        bad = nwc.nwc_info()
        nwc.nwc_prefill_workspace_size(bad)


def test_gather_validation():
    L = nwc._lib
    blob = nwc.nwc_encode(workloads.gaussian_bits((64, 512), 0.02, 2))
    info = nwc.nwc_inspect(blob)
    A = 1 << 20
    ok = ctypes.c_void_p(A)
    call = lambda ids=ok, n=4, out=ok, ld=512: L.nwc_gather_rows(ctypes.byref(info), ok, ids, n, out, ld, None)
    assert call(ids=None) == nwc.NWC_ERR_INVALID_ARG
    assert call(out=None) == nwc.NWC_ERR_INVALID_ARG
    assert call(n=0) == nwc.NWC_ERR_INVALID_ARG
    assert call(ld=511) == nwc.NWC_ERR_INVALID_ARG
    assert call(out=ctypes.c_void_p(A + 1)) == nwc.NWC_ERR_ALIGNMENT
    assert call(ids=ctypes.c_void_p(A + 2)) == nwc.NWC_ERR_ALIGNMENT
    assert L.nwc_gather_rows(ctypes.byref(info), ctypes.c_void_p(A + 8), ok, 4, ok, 512, None) == nwc.NWC_ERR_ALIGNMENT



def test_one_hip_runtime_whatever_the_import_order():
    # importing the package before torch must not map a second HIP (or HSA)
    # runtime beside torch's own copy
    code = ("import decode_gemv_byte_amd, torch\n"
            "m = open('/proc/self/maps').read().splitlines()\n"
            "print(sorted({l.split()[-1] for l in m if 'libamdhip64' in l}))\n"
            "print(sorted({l.split()[-1] for l in m if 'libhsa-runtime64' in l}))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert out.returncode == 0, out.stderr
    hip, hsa = [eval(l) for l in out.stdout.strip().splitlines()[-2:]]
    assert len(hip) == 1 and len(hsa) == 1, (hip, hsa)


@pytest.mark.parametrize("pair_fit", [64, 1024])
@pytest.mark.parametrize("cid,name", [(1, "w"), (2, "q"), (2, "down"), (3, "gate"), (5, "lm_head")])
def test_encoder_bytes_equal_oracle_pair_fit(cid, name, pair_fit):
    w = workloads.weights(cid, name)
    if w.shape[0] > 4096:
        w = np.ascontiguousarray(w[:4096])
    blob = nwc.nwc_encode(w, dict(pair_fit=pair_fit))
    assert np.array_equal(blob, oracle.encode(w, 8, 512, 64, 8, pair_fit))
    info = nwc.nwc_inspect(blob)
    e, _ = oracle.split(w)
    h = oracle.histogram(e)
    common = h * pair_fit >= h.sum()
    assert np.all(np.asarray(info.code_len)[common] <= 6)
    assert np.array_equal(oracle.decode(blob), w)


def test_pair_fit_infeasible_caps_fall_back_like_the_oracle():
    w = workloads.random_bits((64, 64), 3)     # ~1/256 of the weights per exponent value
    # all 256 values would be capped at 6 bits, which no prefix code allows:
    # both sides fall back to the plain limit
    blob = nwc.nwc_encode(w, dict(pair_fit=1024))
    assert np.array_equal(blob, oracle.encode(w, 8, 512, 64, 8, 1024))
    assert np.array_equal(blob, oracle.encode(w, 8, 512, 64, 8, 1))
    assert np.array_equal(nwc.nwc_encode(w, dict(pair_fit=128)), oracle.encode(w, 8, 512, 64, 8, 128))
    # pair_fit 1 caps nothing: the plain limit
    w2 = workloads.weights(1, "w")
    assert np.array_equal(nwc.nwc_encode(w2, dict(pair_fit=1)), oracle.encode(w2, 8, 512, 64, 8, 0))


@pytest.mark.parametrize("lmax", [8, 12])
@pytest.mark.parametrize("cid,name", [(1, "w"), (2, "gate"), (3, "gate"), (5, "lm_head"), (0, "all_patterns"),
                                      (0, "one_symbol")])
def test_encoder_bytes_equal_oracle_unary_family(cid, name, lmax):
    # the ranked unary code with an escape (code_family 1): the library's
    # lengths, canonical codes and blob bytes are the oracle's
    if cid == 0:
        w = workloads.all_patterns() if name == "all_patterns" else np.full((40, 72), 0x3C55, np.uint16)
    else:
        w = workloads.weights(cid, name, rows=slice(0, 2048))
    blob = nwc.nwc_encode(w, dict(max_code_len=lmax, code_family=1))
    assert np.array_equal(blob, oracle.encode(w, 8, 512, 64, lmax, 0, family=1))
    info = nwc.nwc_inspect(blob)
    e, _ = oracle.split(w)
    assert np.array_equal(np.asarray(info.code_len), oracle.code_lengths_unary(oracle.histogram(e), lmax))
    assert np.array_equal(oracle.decode(blob), w)


def test_unknown_code_family_is_rejected():
    w = workloads.gaussian_bits((16, 512), 0.02, 1)
    with pytest.raises(nwc.NwcError):
        nwc.nwc_encode(w, dict(code_family=2))


def _device_metadata():
    """The AMDGPU kernel metadata of the built library's gfx950 code object
    (section .hip_fatbin, unbundled, notes read), as parsed YAML; None when
    the ROCm LLVM tools are not there."""
    import shutil
    import subprocess
    import tempfile
    import yaml
    tools = "/opt/rocm/llvm/bin"
    objcopy, bundler, readelf = (os.path.join(tools, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf"))
    if not all(os.path.exists(t) for t in (objcopy, bundler, readelf)):
        return None
    lib = os.path.join(ROOT, "decode_gemv_byte_amd", "libnwc.so")
    with tempfile.TemporaryDirectory() as d:
        fb, co = os.path.join(d, "fb.bin"), os.path.join(d, "co.o")
        shutil.copy(lib, os.path.join(d, "lib.so"))
        subprocess.run([objcopy, "--dump-section", ".hip_fatbin=" + fb, os.path.join(d, "lib.so"),
                        os.path.join(d, "out.so")], check=True, capture_output=True)
        subprocess.run([bundler, "--unbundle", "--type=o", "--input=" + fb,
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", "--output=" + co], check=True, capture_output=True)
        notes = subprocess.run([readelf, "--notes", co], check=True, capture_output=True, text=True).stdout
    text = notes[notes.index("---"):]
    text = text[text.index("\n") + 1:text.index("\n...")]
    return yaml.safe_load(text)


def test_k_gemv_argument_layout():
    # k_gemv reads its group argument through the kernel-argument segment at
    # a fixed byte offset (after seven 32-bit arguments that the build
    # preloads into scalar registers): every k_gemv in the built code object
    # must have the group at exactly that offset, and the seven arguments
    # before it (a wrong offset reads garbage pointers on the GPU)
    meta = _device_metadata()
    if meta is None:
        pytest.skip("ROCm LLVM tools not found")
    kernels = [k for k in meta["amdhsa.kernels"] if k[".name"].startswith("_ZN12_GLOBAL__N_16k_gemvI")]
    assert len(kernels) >= 30
    for k in kernels:
        args = k[".args"]
        assert [a[".offset"] for a in args[:7]] == [0, 4, 8, 12, 16, 20, 24], k[".name"]
        assert all(a[".size"] == 4 for a in args[:7]), k[".name"]
        assert args[7][".offset"] == 32 and args[7][".size"] > 1000, k[".name"]
        assert k[".kernarg_segment_size"] >= 32 + args[7][".size"]
