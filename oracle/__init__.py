"""CPU oracle for compressed-BF16 decode and decode-GEMV -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and this
package imports nothing from the product: the two share no code.

The arithmetic lives in ``nwc_oracle.c`` (plain scalar C, FP64 for the
products), compiled with gcc into ``oracle/_build/``; this module only
marshals numpy arrays.  See the C file's header for the sources each step
follows and for the blob layout.
"""
from __future__ import annotations

import ctypes
import math
import os
import struct
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nwc_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "libnwc_oracle.so")

OK, EINVAL, ESMALL, EFORMAT = 0, -1, -2, -3
HEADER_BYTES = 256
TABLE_ENTRIES = 4096

_lib: Optional[ctypes.CDLL] = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C11, -O2, no fast-math)."""
    os.makedirs(_BUILD, exist_ok=True)
    stale = not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = build()
        L = ctypes.CDLL(path)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        u64p = ctypes.POINTER(ctypes.c_uint64)
        f64p = ctypes.POINTER(ctypes.c_double)
        u64 = ctypes.c_uint64
        u32 = ctypes.c_uint32
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_split.argtypes = [u16p, u64, u8p, u8p]
        L.orc_join.argtypes = [u8p, u8p, u64, u16p]
        L.orc_histogram.argtypes = [u8p, u64, u64p]
        L.orc_code_lengths.argtypes = [u64p, ctypes.c_int, u8p]
        L.orc_code_lengths_pair_fit.argtypes = [u64p, ctypes.c_int, u32, u8p]
        L.orc_code_lengths_unary.argtypes = [u64p, ctypes.c_int, u8p]
        L.orc_canonical_codes.argtypes = [u8p, u16p]
        L.orc_decode_table.argtypes = [u8p, u32p]
        L.orc_encode_bound.argtypes = [u64, u64, u32, u32, u32, u32, u64p]
        L.orc_encode.argtypes = [u16p, u64, u64, u64, u32, u32, u32, u32, u32, u8p, u64, u64p]
        L.orc_encode_family.argtypes = [u16p, u64, u64, u64, u32, u32, u32, u32, u32, u32, u8p, u64, u64p]
        L.orc_decode.argtypes = [u8p, u64, u16p, u64]
        L.orc_decode_chunk.argtypes = [u8p, u64, u64, u32, u8p, u64]
        L.orc_decode_chunk.restype = ctypes.c_int64
        L.orc_validate.argtypes = [u8p, u64]
        L.orc_gemv.argtypes = [u16p, u64, u64, u64, u16p, f64p, f64p]
        L.orc_gemv.restype = None
        L.orc_gemm.argtypes = [u16p, u64, u64, u64, u16p, u64, u64, f64p, f64p]
        L.orc_gemm.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("expected uint16 BF16 bit patterns, got %s" % a.dtype)
    return a


# ---------------------------------------------------------------- planes ---

def bf16_value(bits) -> np.ndarray:
    """FP64 value of each BF16 pattern, from the sign/exponent/fraction definition."""
    b = _u16(np.asarray(bits)).ravel()
    L = lib()
    out = np.empty(b.size, np.float64)
    for i, v in enumerate(b.tolist()):
        out[i] = L.orc_bf16_value(v)
    return out.reshape(np.shape(bits))


def split(w) -> Tuple[np.ndarray, np.ndarray]:
    w = _u16(w)
    e = np.empty(w.shape, np.uint8)
    r = np.empty(w.shape, np.uint8)
    lib().orc_split(_p(w, ctypes.c_uint16), w.size, _p(e, ctypes.c_uint8), _p(r, ctypes.c_uint8))
    return e, r


def join(e, r) -> np.ndarray:
    e = np.ascontiguousarray(e, np.uint8)
    r = np.ascontiguousarray(r, np.uint8)
    if e.shape != r.shape:
        raise ValueError("plane shapes differ")
    w = np.empty(e.shape, np.uint16)
    lib().orc_join(_p(e, ctypes.c_uint8), _p(r, ctypes.c_uint8), e.size, _p(w, ctypes.c_uint16))
    return w


def histogram(e) -> np.ndarray:
    e = np.ascontiguousarray(e, np.uint8)
    h = np.zeros(256, np.uint64)
    lib().orc_histogram(_p(e, ctypes.c_uint8), e.size, _p(h, ctypes.c_uint64))
    return h


def entropy_bits(h) -> float:
    """Shannon entropy (bits/symbol) of a histogram."""
    h = np.asarray(h, np.float64)
    tot = h.sum()
    p = h[h > 0] / tot
    return float(-(p * np.log2(p)).sum())


# ------------------------------------------------------------------ code ---

def code_lengths(h, lmax: int, pair_fit: int = 0) -> np.ndarray:
    """Optimal prefix-code lengths of at most lmax bits; with pair_fit > 0 the
    symbols holding at least 1/pair_fit of the counts are capped at 6 bits."""
    h = np.ascontiguousarray(h, np.uint64)
    if h.shape != (256,):
        raise ValueError("histogram must have 256 bins")
    out = np.zeros(256, np.uint8)
    rc = lib().orc_code_lengths_pair_fit(_p(h, ctypes.c_uint64), int(lmax), ctypes.c_uint32(int(pair_fit)),
                                         _p(out, ctypes.c_uint8))
    if rc:
        raise ValueError("code_lengths failed (%d)" % rc)
    return out


def code_lengths_unary(h, lmax: int) -> np.ndarray:
    """Lengths of the ranked unary code with an escape of at most lmax bits
    (see orc_code_lengths_unary)."""
    h = np.ascontiguousarray(h, np.uint64)
    if h.shape != (256,):
        raise ValueError("histogram must have 256 bins")
    out = np.zeros(256, np.uint8)
    rc = lib().orc_code_lengths_unary(_p(h, ctypes.c_uint64), int(lmax), _p(out, ctypes.c_uint8))
    if rc:
        raise ValueError("code_lengths_unary failed (%d)" % rc)
    return out


def canonical_codes(lengths) -> np.ndarray:
    ln = np.ascontiguousarray(lengths, np.uint8)
    out = np.zeros(256, np.uint16)
    rc = lib().orc_canonical_codes(_p(ln, ctypes.c_uint8), _p(out, ctypes.c_uint16))
    if rc:
        raise ValueError("lengths over-subscribe the code space")
    return out


def decode_table(lengths) -> np.ndarray:
    ln = np.ascontiguousarray(lengths, np.uint8)
    out = np.zeros(TABLE_ENTRIES, np.uint32)
    lib().orc_decode_table(_p(ln, ctypes.c_uint8), _p(out, ctypes.c_uint32))
    return out


# ------------------------------------------------------------------ blob ---

def encode_bound(rows, cols, tile_rows, tile_cols, chunks_per_tile, max_code_len) -> int:
    b = ctypes.c_uint64(0)
    rc = lib().orc_encode_bound(rows, cols, tile_rows, tile_cols, chunks_per_tile,
                                max_code_len, ctypes.byref(b))
    if rc:
        raise ValueError("invalid geometry (%d)" % rc)
    return b.value


def encode(w, tile_rows: int, tile_cols: int, chunks_per_tile: int,
           max_code_len: int, pair_fit: int = 0, family: int = 0) -> np.ndarray:
    """Encode a 2-D uint16 BF16 matrix into a blob (uint8 array); pair_fit > 0
    caps the codes of exponents with at least 1/pair_fit of the weights at 6
    bits (see code_lengths); family 1 takes the ranked unary code with an
    escape instead (see code_lengths_unary)."""
    w = _u16(w)
    if w.ndim != 2:
        raise ValueError("expected a 2-D matrix")
    rows, cols = w.shape
    cap = encode_bound(rows, cols, tile_rows, tile_cols, chunks_per_tile, max_code_len)
    blob = np.zeros(cap, np.uint8)
    used = ctypes.c_uint64(0)
    rc = lib().orc_encode_family(_p(w, ctypes.c_uint16), rows, cols, cols, tile_rows, tile_cols,
                                 chunks_per_tile, max_code_len, int(pair_fit), int(family),
                                 _p(blob, ctypes.c_uint8), cap, ctypes.byref(used))
    if rc:
        raise ValueError("encode failed (%d)" % rc)
    return blob[: used.value].copy()


def header(blob) -> dict:
    b = bytes(np.asarray(blob, np.uint8)[:HEADER_BYTES])
    magic, version, hbytes = struct.unpack_from("<IHH", b, 0)
    rows, cols = struct.unpack_from("<QQ", b, 8)
    tr, tc, s, lmax, kind, flags = struct.unpack_from("<6I", b, 24)
    names = ["raw_ld", "n_tiles", "n_chunks", "stream_words", "off_code_len", "off_table",
             "off_tile_words", "off_chunk_bits", "off_raw", "off_stream", "total_bytes"]
    vals = struct.unpack_from("<11Q", b, 48)
    d = dict(magic=magic, version=version, header_bytes=hbytes, rows=rows, cols=cols,
             tile_rows=tr, tile_cols=tc, chunks_per_tile=s, max_code_len=lmax,
             table_kind=kind, flags=flags)
    d.update(zip(names, vals))
    return d


def sections(blob) -> dict:
    """Views of the blob's sections (code lengths, table, offsets, raw, stream)."""
    blob = np.asarray(blob, np.uint8)
    h = header(blob)
    d = {}
    d["code_len"] = blob[h["off_code_len"]: h["off_code_len"] + 256]
    d["table"] = blob[h["off_table"]: h["off_table"] + 4 * TABLE_ENTRIES].view(np.uint32)
    d["tile_words"] = blob[h["off_tile_words"]: h["off_tile_words"] + 4 * (h["n_tiles"] + 1)].view(np.uint32)
    d["chunk_bits"] = blob[h["off_chunk_bits"]: h["off_chunk_bits"] + 2 * h["n_chunks"]].view(np.uint16)
    d["raw"] = blob[h["off_raw"]: h["off_raw"] + h["raw_ld"] * h["rows"]].reshape(h["rows"], h["raw_ld"])
    d["stream"] = blob[h["off_stream"]: h["off_stream"] + 4 * h["stream_words"]].view(np.uint32)
    return d


def validate(blob) -> int:
    blob = np.ascontiguousarray(blob, np.uint8)
    return lib().orc_validate(_p(blob, ctypes.c_uint8), blob.size)


def decode(blob) -> np.ndarray:
    blob = np.ascontiguousarray(blob, np.uint8)
    h = header(blob) if blob.size >= HEADER_BYTES else None
    if h is None or h["rows"] * h["cols"] > (1 << 34):
        raise ValueError("not a blob")
    w = np.zeros((h["rows"], h["cols"]), np.uint16)
    rc = lib().orc_decode(_p(blob, ctypes.c_uint8), blob.size, _p(w, ctypes.c_uint16), h["cols"])
    if rc:
        raise ValueError("decode failed (%d)" % rc)
    return w


def decode_chunk(blob, tile: int, chunk: int) -> np.ndarray:
    blob = np.ascontiguousarray(blob, np.uint8)
    h = header(blob)
    cap = h["tile_rows"] * (h["tile_cols"] // h["chunks_per_tile"])
    out = np.zeros(max(cap, 1), np.uint8)
    k = lib().orc_decode_chunk(_p(blob, ctypes.c_uint8), blob.size, tile, chunk,
                               _p(out, ctypes.c_uint8), out.size)
    if k < 0:
        raise ValueError("decode_chunk failed (%d)" % k)
    return out[:k].copy()


# -------------------------------------------------------------- products ---

def gemv(w, x) -> Tuple[np.ndarray, np.ndarray]:
    """FP64 y = W x and a = |W| |x| (elementwise magnitudes) for BF16 patterns."""
    w = _u16(w)
    x = _u16(np.asarray(x).ravel())
    rows, cols = w.shape
    if x.size != cols:
        raise ValueError("x has %d entries, W has %d columns" % (x.size, cols))
    y = np.zeros(rows, np.float64)
    a = np.zeros(rows, np.float64)
    lib().orc_gemv(_p(w, ctypes.c_uint16), rows, cols, cols, _p(x, ctypes.c_uint16),
                   _p(y, ctypes.c_double), _p(a, ctypes.c_double))
    return y, a


def gemm(w, X) -> Tuple[np.ndarray, np.ndarray]:
    """FP64 Y[b] = W X[b] for each batch row of X; returns (Y, A), both [batch, rows]."""
    w = _u16(w)
    X = _u16(X)
    rows, cols = w.shape
    batch = X.shape[0]
    if X.shape[1] != cols:
        raise ValueError("X has %d columns, W has %d" % (X.shape[1], cols))
    Y = np.zeros((batch, rows), np.float64)
    A = np.zeros((batch, rows), np.float64)
    lib().orc_gemm(_p(w, ctypes.c_uint16), rows, cols, cols, _p(X, ctypes.c_uint16), batch,
                   cols, _p(Y, ctypes.c_double), _p(A, ctypes.c_double))
    return Y, A


def gemv_rows(w, x, row_idx) -> Tuple[np.ndarray, np.ndarray]:
    """FP64 y and a for selected rows only (for sampled checks at full size)."""
    w = _u16(w)
    idx = np.asarray(row_idx, np.int64)
    sub = np.ascontiguousarray(w[idx])
    return gemv(sub, x)


def size_report(blob) -> dict:
    """Bits per weight of the exponent side (header, lengths, table, offsets,
    stream) and of the raw plane, next to the exponent entropy."""
    blob = np.asarray(blob, np.uint8)
    h = header(blob)
    n = h["rows"] * h["cols"]
    sec = sections(blob)
    exp_bytes = blob.size - h["raw_ld"] * h["rows"]
    payload_bits = int(sec["chunk_bits"].astype(np.uint64).sum())
    return dict(weights=n, blob_bytes=int(blob.size), exp_bits_per_weight=8.0 * exp_bytes / n,
                payload_bits_per_weight=payload_bits / n,
                bytes_per_weight=blob.size / n)
