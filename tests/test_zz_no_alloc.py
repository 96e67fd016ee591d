"""nwc_gemv_noalloc (no workspace: a static per-device scratch array) gives the
same bits as nwc_gemv with a caller's workspace, on two calls in a row, the
second with a smaller matrix, in FP32 and BF16 output; it rejects what it
cannot run without enqueuing anything."""
import ctypes
import sys

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
import decode_gemv_byte_amd as nwc  # noqa: E402

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(w, seed):
    host = nwc.nwc_encode(w)
    info = nwc.nwc_inspect(host)
    x = workloads.gaussian_bits((w.shape[1],), 1.0, seed)
    return info, dev(host), dev(x)


@pytest.mark.parametrize("out_f32", [True, False])
def test_noalloc_equals_workspace_call(out_f32):
    dt = torch.float32 if out_f32 else torch.bfloat16
    iv = torch.int32 if out_f32 else torch.int16
    big = _case(workloads.weights(3, "gate"), 81)                  # 14336 x 4096, cut row blocks
    small = _case(workloads.gaussian_bits((1000, 2560), 0.02, 82), 83)
    for name, (info, blob, x) in (("big", big), ("small", small), ("big again", big)):
        _say("noalloc %s %dx%d f32=%s" % (name, info.rows, info.cols, out_f32))
        ws = torch.zeros(nwc.nwc_workspace_size(info, 1), dtype=torch.uint8, device="cuda")
        want = torch.empty(info.rows, dtype=dt, device="cuda")
        nwc.nwc_gemv(info, blob, x, want, ws)
        got = torch.full((info.rows,), 7.0, dtype=dt, device="cuda")
        nwc.nwc_gemv_noalloc(info, blob, x, got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(iv), want.view(iv)), name


def test_noalloc_rejects_before_launch():
    # host-side refusals (these calls enqueue nothing)
    L = nwc._lib
    A = 0x10000
    odd = nwc.nwc_inspect(nwc.nwc_encode(workloads.gaussian_bits((64, 500), 0.02, 2)))   # generic geometry
    assert L.nwc_gemv_noalloc(ctypes.byref(odd), A, A, A, 0, None) == nwc.NWC_ERR_UNSUPPORTED
    ok = nwc.nwc_inspect(nwc.nwc_encode(workloads.gaussian_bits((64, 512), 0.02, 2)))
    assert L.nwc_gemv_noalloc(None, A, A, A, 0, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv_noalloc(ctypes.byref(ok), A, A, None, 0, None) == nwc.NWC_ERR_INVALID_ARG
    assert L.nwc_gemv_noalloc(ctypes.byref(ok), A, A + 2, A, 0, None) == nwc.NWC_ERR_ALIGNMENT
    # a matrix whose slots exceed the scratch: (2^21 + 8) x 512 at 8-row
    # tiles has 2^18 + 1 tiles of 64 slot bytes each.  Described by its
    # header fields (the blob layout of the format: 256-byte header, code
    # lengths, decode table, tile offsets, chunk lengths, raw plane, stream),
    # not encoded.
    assert nwc.nwc_noalloc_scratch_bytes() == 16 << 20
    up = lambda v, a: -(-v // a) * a
    rows, cols, words = (1 << 21) + 8, 512, 1000
    big = nwc.nwc_info.from_buffer_copy(ok)
    big.rows, big.cols = rows, cols
    big.n_tiles = rows // 8
    big.n_chunks = big.n_tiles * 64
    big.raw_ld = up(cols, 16)
    big.stream_words = words
    big.off_code_len = 256
    big.off_table = 512
    big.off_tile_words = 512 + 4 * 4096
    big.off_chunk_bits = up(big.off_tile_words + 4 * (big.n_tiles + 1), 256)
    big.off_raw = up(big.off_chunk_bits + 2 * big.n_chunks, 256)
    big.off_stream = up(big.off_raw + big.raw_ld * rows, 256)
    big.blob_bytes = up(big.off_stream + 4 * words + 16, 256)
    assert nwc.nwc_workspace_size(big, 1) > 16 << 20
    assert L.nwc_gemv_noalloc(ctypes.byref(big), A, A, A, 0, None) == nwc.NWC_ERR_SCRATCH_LIMIT
    assert nwc.nwc_status_str(nwc.NWC_ERR_SCRATCH_LIMIT) == "NWC_ERR_SCRATCH_LIMIT"
