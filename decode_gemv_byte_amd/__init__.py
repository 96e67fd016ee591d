"""Python binding of libnwc -- lossless BF16 weight compression decoded inside
the matrix-vector kernel, for MI355X (gfx950).

Argument marshalling only: every step runs in the native library
(``libnwc.so``: C++ host codec + HIP kernels).  The functions carry the names
of the C ABI in ``include/nwc.h``.  Host buffers are numpy arrays; device
buffers are torch CUDA tensors (PyTorch provides device memory and streams).
Importing fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnwc.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libnwc.so is not built; run `python decode_gemv_byte_amd/build.py` "
                      "(or __graft_entry__.build())")

# The binding hands torch tensors' device memory and streams to the library,
# so both must run on one HIP runtime.  PyTorch ships its own copy of it;
# with torch loaded first, the library's dependency on the runtime's soname
# resolves to that copy.  Loaded the other way round, the library would map
# the ROCm install's runtime and torch would then map its own beside it: two
# runtimes (and two HSA runtimes) in one process, under which torch's
# streams and allocations are foreign handles and launches fail.
try:
    import torch  # noqa: F401
except ImportError:   # a torch-free caller of the C ABI: the ROCm install's runtime
    pass

_lib = ctypes.CDLL(LIB_PATH)

NWC_OK = 0
NWC_ERR_INVALID_ARG = -1
NWC_ERR_BUFFER_TOO_SMALL = -2
NWC_ERR_BAD_FORMAT = -3
NWC_ERR_UNSUPPORTED = -4
NWC_ERR_ALIGNMENT = -5
NWC_ERR_HIP = -6
NWC_ERR_SCRATCH_LIMIT = -7
NWC_OUT_BF16 = 0
NWC_OUT_F32 = 1


class nwc_params(ctypes.Structure):
    _fields_ = [("tile_rows", ctypes.c_uint32), ("tile_cols", ctypes.c_uint32),
                ("chunks_per_tile", ctypes.c_uint32), ("max_code_len", ctypes.c_uint32),
                ("pair_fit", ctypes.c_uint32), ("code_family", ctypes.c_uint32)]


class nwc_info(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_uint64), ("cols", ctypes.c_uint64), ("blob_bytes", ctypes.c_uint64),
                ("tile_rows", ctypes.c_uint32), ("tile_cols", ctypes.c_uint32),
                ("chunks_per_tile", ctypes.c_uint32), ("max_code_len", ctypes.c_uint32),
                ("n_tiles", ctypes.c_uint64), ("n_chunks", ctypes.c_uint64), ("raw_ld", ctypes.c_uint64),
                ("stream_words", ctypes.c_uint64), ("off_code_len", ctypes.c_uint64),
                ("off_table", ctypes.c_uint64), ("off_tile_words", ctypes.c_uint64),
                ("off_chunk_bits", ctypes.c_uint64), ("off_raw", ctypes.c_uint64),
                ("off_stream", ctypes.c_uint64), ("max_tile_words", ctypes.c_uint32),
                ("n_symbols", ctypes.c_uint32), ("max_chunk_bits", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32), ("payload_bits", ctypes.c_uint64),
                ("code_len", ctypes.c_uint8 * 256)]


class NwcError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s" % (where, nwc_status_str(status)))


_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_u64 = ctypes.c_uint64
_u32 = ctypes.c_uint32
_i = ctypes.c_int
_st = ctypes.c_int

_lib.nwc_status_str.argtypes = [_st]
_lib.nwc_status_str.restype = ctypes.c_char_p
_lib.nwc_encode_bound.argtypes = [_u64, _u64, ctypes.POINTER(nwc_params), ctypes.POINTER(_sz)]
_lib.nwc_encode.argtypes = [_vp, _u64, _u64, _u64, ctypes.POINTER(nwc_params), _vp, _sz, ctypes.POINTER(_sz)]
_lib.nwc_inspect.argtypes = [_vp, _sz, ctypes.POINTER(nwc_info)]
_lib.nwc_decode.argtypes = [ctypes.POINTER(nwc_info), _vp, _vp, _u64, _vp]
_lib.nwc_workspace_size.argtypes = [ctypes.POINTER(nwc_info), _i, ctypes.POINTER(_sz)]
_lib.nwc_gemv.argtypes = [ctypes.POINTER(nwc_info), _vp, _vp, _vp, _i, _vp, _sz, _vp]
_lib.nwc_gemm_skinny.argtypes = [ctypes.POINTER(nwc_info), _vp, _vp, _u64, _i, _vp, _u64, _i, _vp, _sz, _vp]
_lib.nwc_bf16_workspace_size.argtypes = [_u64, _u64, ctypes.POINTER(_sz)]
_lib.nwc_gemv_bf16.argtypes = [_vp, _u64, _u64, _u64, _vp, _vp, _i, _vp, _sz, _vp]
_lib.nwc_gemv_batched.argtypes = [_i, ctypes.POINTER(nwc_info), ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                  ctypes.POINTER(_vp), _i, _vp, _sz, _vp]
_lib.nwc_decode_batched.argtypes = [_i, ctypes.POINTER(nwc_info), ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                    ctypes.POINTER(_u64), _vp]
_lib.nwc_gather_rows.argtypes = [ctypes.POINTER(nwc_info), _vp, _vp, _u32, _vp, _u64, _vp]
_lib.nwc_blas_create.argtypes = [ctypes.POINTER(_vp)]
_lib.nwc_blas_destroy.argtypes = [_vp]
_lib.nwc_prefill_workspace_size.argtypes = [ctypes.POINTER(nwc_info), ctypes.POINTER(_sz)]
_lib.nwc_gemm_prefill.argtypes = [_vp, ctypes.POINTER(nwc_info), _vp, _vp, _u64, _i, _vp, _u64, _i, _vp, _sz, _vp]
_lib.nwc_read_probe.argtypes = [_vp, _sz, _vp, _u32, _i, _vp]
_lib.nwc_noalloc_scratch_bytes.argtypes = [ctypes.POINTER(_sz)]
_lib.nwc_gemv_noalloc.argtypes = [ctypes.POINTER(nwc_info), _vp, _vp, _vp, _i, _vp]
_lib.nwc_set_wait_limit.argtypes = [_u32]
for _f in ("nwc_encode_bound", "nwc_encode", "nwc_inspect", "nwc_decode", "nwc_workspace_size", "nwc_gemv",
           "nwc_gemm_skinny", "nwc_bf16_workspace_size", "nwc_gemv_bf16", "nwc_gemv_batched", "nwc_decode_batched",
           "nwc_blas_create", "nwc_blas_destroy", "nwc_prefill_workspace_size", "nwc_gemm_prefill",
           "nwc_gather_rows", "nwc_read_probe", "nwc_noalloc_scratch_bytes", "nwc_gemv_noalloc",
           "nwc_set_wait_limit"):
    getattr(_lib, _f).restype = _st

# the exported C symbols, for checks against include/nwc.h
EXPORTS = ("nwc_status_str", "nwc_encode_bound", "nwc_encode", "nwc_inspect", "nwc_decode",
           "nwc_workspace_size", "nwc_gemv", "nwc_gemm_skinny", "nwc_bf16_workspace_size", "nwc_gemv_bf16",
           "nwc_gemv_batched", "nwc_decode_batched", "nwc_blas_create", "nwc_blas_destroy",
           "nwc_prefill_workspace_size", "nwc_gemm_prefill", "nwc_gather_rows", "nwc_read_probe",
           "nwc_noalloc_scratch_bytes", "nwc_gemv_noalloc", "nwc_set_wait_limit")


def _check(st: int, where: str):
    if st != NWC_OK:
        raise NwcError(st, where)


def _params(p) -> Optional[nwc_params]:
    if p is None:
        return None
    if isinstance(p, nwc_params):
        return p
    return nwc_params(*[int(p.get(k, 0)) for k in ("tile_rows", "tile_cols", "chunks_per_tile",
                                                    "max_code_len", "pair_fit", "code_family")])


def _ptr_params(p):
    return ctypes.byref(p) if p is not None else None


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dptr(t, rows: bool = False) -> ctypes.c_void_p:
    """Device address of a tensor: contiguous, or with rows=True a 2-D tensor
    whose rows are contiguous and may sit any stride(0) apart."""
    if hasattr(t, "data_ptr"):
        if not t.is_cuda:
            raise ValueError("expected a device (cuda) tensor")
        if rows and t.dim() == 2 and t.stride(1) == 1:
            return ctypes.c_void_p(t.data_ptr())
        if not t.is_contiguous():
            raise ValueError("expected a contiguous tensor")
        return ctypes.c_void_p(t.data_ptr())
    return ctypes.c_void_p(int(t))


def _ytype(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return NWC_OUT_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return NWC_OUT_BF16
    raise ValueError("y must be float32 or bfloat16")


# ------------------------------------------------------------------ host ---

def nwc_status_str(status: int) -> str:
    return _lib.nwc_status_str(int(status)).decode()


def nwc_encode_bound(rows: int, cols: int, params=None) -> int:
    p = _params(params)
    out = _sz(0)
    _check(_lib.nwc_encode_bound(rows, cols, _ptr_params(p), ctypes.byref(out)), "nwc_encode_bound")
    return out.value


def nwc_encode(w: np.ndarray, params=None) -> np.ndarray:
    """Encode a 2-D uint16 (BF16 bit pattern) matrix into a blob (uint8 array)."""
    if w.dtype != np.uint16 or w.ndim != 2:
        raise ValueError("expected a 2-D uint16 array of BF16 bit patterns")
    if w.strides[1] != 2 or w.strides[0] % 2:
        w = np.ascontiguousarray(w)
    rows, cols = w.shape
    ld = w.strides[0] // 2
    p = _params(params)
    cap = nwc_encode_bound(rows, cols, p)
    blob = np.empty(cap, np.uint8)
    used = _sz(0)
    _check(_lib.nwc_encode(w.ctypes.data, rows, cols, ld, _ptr_params(p), blob.ctypes.data, cap,
                           ctypes.byref(used)), "nwc_encode")
    return blob[: used.value]


def nwc_inspect(blob: np.ndarray) -> nwc_info:
    blob = np.ascontiguousarray(blob, np.uint8)
    info = nwc_info()
    _check(_lib.nwc_inspect(blob.ctypes.data, blob.size, ctypes.byref(info)), "nwc_inspect")
    return info


def nwc_workspace_size(info: nwc_info, batch: int = 1) -> int:
    out = _sz(0)
    _check(_lib.nwc_workspace_size(ctypes.byref(info), batch, ctypes.byref(out)), "nwc_workspace_size")
    return out.value


def nwc_bf16_workspace_size(rows: int, cols: int) -> int:
    out = _sz(0)
    _check(_lib.nwc_bf16_workspace_size(rows, cols, ctypes.byref(out)), "nwc_bf16_workspace_size")
    return out.value


# ---------------------------------------------------------------- device ---

def nwc_decode(info: nwc_info, blob_dev, w_dev, ld: Optional[int] = None, stream=None):
    """Decode into w_dev (device uint16/bfloat16, rows x ld)."""
    if ld is None:
        ld = int(w_dev.shape[-1])
    _check(_lib.nwc_decode(ctypes.byref(info), _dptr(blob_dev), _dptr(w_dev), ld, _stream(stream)), "nwc_decode")


class DecodeBatch:
    """Marshalled arguments of one nwc_decode_batched call (blobs i written to
    w_devs[i], row stride = its last dimension), built once and reusable."""

    def __init__(self, infos: Sequence[nwc_info], blobs_dev, w_devs):
        n = len(infos)
        if not (n == len(blobs_dev) == len(w_devs)) or n < 1:
            raise ValueError("need equal, non-empty lists")
        self.count = n
        self.infos = (nwc_info * n)(*infos)
        self.blobs = (_vp * n)(*[_dptr(t).value for t in blobs_dev])
        self.outs = (_vp * n)(*[_dptr(t).value for t in w_devs])
        self.ld = (_u64 * n)(*[int(t.shape[-1]) for t in w_devs])
        self._keep = (list(blobs_dev), list(w_devs))


def nwc_decode_batched(batch: DecodeBatch, stream=None):
    """Several independent decodes in one launch."""
    _check(_lib.nwc_decode_batched(batch.count, batch.infos, batch.blobs, batch.outs, batch.ld, _stream(stream)),
           "nwc_decode_batched")


def _ws(ws):
    if ws is None:
        return ctypes.c_void_p(None), 0
    return _dptr(ws), ws.numel() * ws.element_size()


def nwc_gemv(info: nwc_info, blob_dev, x_dev, y_dev, ws=None, stream=None):
    """y = W x; y_dev float32 or bfloat16 (rows); ws a device byte tensor of
    nwc_workspace_size(info, 1) bytes (zero-filled before its first use on the
    fused path), or None when that size is 0."""
    wp, wn = _ws(ws)
    _check(_lib.nwc_gemv(ctypes.byref(info), _dptr(blob_dev), _dptr(x_dev), _dptr(y_dev), _ytype(y_dev),
                         wp, wn, _stream(stream)), "nwc_gemv")


def nwc_noalloc_scratch_bytes() -> int:
    out = _sz(0)
    _check(_lib.nwc_noalloc_scratch_bytes(ctypes.byref(out)), "nwc_noalloc_scratch_bytes")
    return out.value


def nwc_set_wait_limit(polls: int = 0):
    """Polls after which the matrix-core skinny GEMM's waits give up (its outputs then NaN); 0 = default."""
    _check(_lib.nwc_set_wait_limit(int(polls)), "nwc_set_wait_limit")


def nwc_gemv_noalloc(info: nwc_info, blob_dev, x_dev, y_dev, stream=None):
    """y = W x like nwc_gemv, with no workspace: the library's static per-device scratch holds the
    exchange slots (calls that overlap on one GPU race)."""
    _check(_lib.nwc_gemv_noalloc(ctypes.byref(info), _dptr(blob_dev), _dptr(x_dev), _dptr(y_dev), _ytype(y_dev),
                                 _stream(stream)), "nwc_gemv_noalloc")


def gemv_batched_workspace_size(infos) -> int:
    """Workspace bytes of one nwc_gemv_batched call over these blobs: the sum
    of their batch-1 workspace sizes."""
    return sum(nwc_workspace_size(i, 1) for i in infos)


class GemvBatch:
    """Marshalled arguments of one nwc_gemv_batched call, built once and reusable
    (e.g. inside a captured graph).  ws is a device byte tensor of at least
    gemv_batched_workspace_size(infos) bytes, zero-filled before its first use.
    Keeps the tensors alive."""

    def __init__(self, infos, blobs_dev, xs_dev, ys_dev, ws):
        n = len(infos)
        if not (n == len(blobs_dev) == len(xs_dev) == len(ys_dev)) or n < 1:
            raise ValueError("need equal, non-empty lists")
        self.count = n
        self.infos = (nwc_info * n)(*infos)
        self.blobs = (_vp * n)(*[_dptr(t).value for t in blobs_dev])
        self.xs = (_vp * n)(*[_dptr(t).value for t in xs_dev])
        self.ys = (_vp * n)(*[_dptr(t).value for t in ys_dev])
        ytypes = {_ytype(t) for t in ys_dev}
        if len(ytypes) != 1:
            raise ValueError("all outputs must have one dtype")
        self.ytype = ytypes.pop()
        self.ws, self.ws_bytes = _ws(ws)
        self._keep = (list(blobs_dev), list(xs_dev), list(ys_dev), ws)


def nwc_gemv_batched(batch: GemvBatch, stream=None):
    """Independent GEMVs y_i = W_i x_i in one launch (see GemvBatch)."""
    _check(_lib.nwc_gemv_batched(batch.count, batch.infos, batch.blobs, batch.xs, batch.ys, batch.ytype,
                                 batch.ws, batch.ws_bytes, _stream(stream)), "nwc_gemv_batched")


def nwc_gemm_skinny(info: nwc_info, blob_dev, X_dev, Y_dev, ws=None, stream=None):
    """Y[b] = W X[b] for X_dev [batch, cols] and Y_dev [batch, rows]."""
    batch = int(X_dev.shape[0])
    wp, wn = _ws(ws)
    _check(_lib.nwc_gemm_skinny(ctypes.byref(info), _dptr(blob_dev), _dptr(X_dev, rows=True), int(X_dev.stride(0)),
                                batch, _dptr(Y_dev, rows=True), int(Y_dev.stride(0)), _ytype(Y_dev), wp, wn,
                                _stream(stream)),
           "nwc_gemm_skinny")


def nwc_gather_rows(info: nwc_info, blob_dev, ids_dev, out_dev, stream=None):
    """out_dev[i] = W[ids_dev[i]] (exact BF16 bits; ids past the matrix give zeros): ids_dev a device
    uint32 / int32 vector, out_dev a device [n, cols] int16 or bfloat16 tensor (rows may be strided)."""
    n = int(ids_dev.numel())
    _check(_lib.nwc_gather_rows(ctypes.byref(info), _dptr(blob_dev), _dptr(ids_dev), n, _dptr(out_dev, rows=True),
                                int(out_dev.stride(0)), _stream(stream)), "nwc_gather_rows")


class Blas:
    """Owns an nwc_blas context (a hipBLASLt handle and its algorithm cache)."""

    def __init__(self):
        h = _vp()
        _check(_lib.nwc_blas_create(ctypes.byref(h)), "nwc_blas_create")
        self.handle = h

    def close(self):
        if self.handle is not None and self.handle.value:
            _check(_lib.nwc_blas_destroy(self.handle), "nwc_blas_destroy")
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def nwc_prefill_workspace_size(info: nwc_info) -> int:
    out = _sz()
    _check(_lib.nwc_prefill_workspace_size(ctypes.byref(info), ctypes.byref(out)), "nwc_prefill_workspace_size")
    return out.value


def nwc_gemm_prefill(blas: Blas, info: nwc_info, blob_dev, X_dev, Y_dev, ws, stream=None):
    """Y[b] = W X[b] for any batch: W decoded into ws, then one hipBLASLt GEMM."""
    batch = int(X_dev.shape[0])
    _check(_lib.nwc_gemm_prefill(blas.handle, ctypes.byref(info), _dptr(blob_dev), _dptr(X_dev, rows=True),
                                 int(X_dev.stride(0)), batch, _dptr(Y_dev, rows=True), int(Y_dev.stride(0)),
                                 _ytype(Y_dev), _dptr(ws),
                                 int(ws.numel() * ws.element_size()), _stream(stream)), "nwc_gemm_prefill")


def nwc_gemv_bf16(w_dev, x_dev, y_dev, ws, stream=None):
    """Uncompressed comparator: y = W x with W a device BF16 matrix [rows, cols]; ws a device byte
    tensor of nwc_bf16_workspace_size(rows, cols) bytes, zero-filled before its first use."""
    rows, cols = int(w_dev.shape[0]), int(w_dev.shape[1])
    wp, wn = _ws(ws)
    _check(_lib.nwc_gemv_bf16(_dptr(w_dev), rows, cols, int(w_dev.stride(0)), _dptr(x_dev), _dptr(y_dev),
                              _ytype(y_dev), wp, wn, _stream(stream)), "nwc_gemv_bf16")


def nwc_read_probe(buf_dev, sink_dev, groups: int = 0, layout: int = 1, stream=None):
    """Stream-read every byte of the device tensor buf_dev (HBM read probe); sink_dev a device tensor
    of at least 4 bytes; layout 0 grid-stride, 1 one contiguous range per workgroup."""
    _check(_lib.nwc_read_probe(_dptr(buf_dev), int(buf_dev.numel() * buf_dev.element_size()), _dptr(sink_dev),
                               int(groups), int(layout), _stream(stream)), "nwc_read_probe")


def info_dict(info: nwc_info) -> dict:
    d = {name: getattr(info, name) for name, _ in nwc_info._fields_ if name != "code_len"}
    d["code_len"] = bytes(info.code_len)
    return d
