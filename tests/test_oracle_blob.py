"""Pins for the oracle's blob writer and decoder (CPU only).

* round trips are bit-exact on every special tensor and on several geometries;
* every chunk decodes on its own, and its symbols are the exponents of exactly
  the block the geometry assigns it (checked with numpy slicing of the matrix);
* the stream of a chunk is the chunk's codes written most significant bit first
  into LSB-first words -- the same convention zlib accepted in the code pins;
* tile offsets are monotone, word aligned and consistent with chunk lengths;
* the exponent side stays within 1 bit/weight of the exponent entropy;
* corrupted blobs are rejected.
"""
import numpy as np
import pytest

import oracle
import workloads

GEOMS = [(16, 512, 64, 12), (32, 512, 64, 12), (8, 256, 32, 12), (1, 64, 8, 12),
         (5, 24, 3, 11), (16, 512, 64, 8), (3, 7, 7, 10)]


def special_tensors():
    rng = np.random.default_rng(5)
    out = {
        "1x1": workloads.gaussian_bits((1, 1), 0.02, 1),
        "1xK": workloads.gaussian_bits((1, 1000), 0.02, 2),
        "Nx1": workloads.gaussian_bits((777, 1), 0.02, 3),
        "127x1001": workloads.gaussian_bits((127, 1001), 0.02, 4),
        "all_zero": np.zeros((64, 96), np.uint16),
        "pm_zero": rng.choice(np.array([0x0000, 0x8000], np.uint16), (40, 50)),
        "nan_payloads": (0x7F80 | rng.integers(1, 128, (33, 65)) |
                         (rng.integers(0, 2, (33, 65)) << 15)).astype(np.uint16),
        "inf": rng.choice(np.array([0x7F80, 0xFF80], np.uint16), (17, 31)),
        "subnormal": (rng.integers(1, 128, (48, 70)) | (rng.integers(0, 2, (48, 70)) << 15)).astype(np.uint16),
        "one_symbol": (0x3C00 | rng.integers(0, 128, (50, 60)) |
                       (rng.integers(0, 2, (50, 60)) << 15)).astype(np.uint16),
        "two_symbol": np.where(rng.random((45, 77)) < 0.9, 0x3C00, 0x4000).astype(np.uint16)
                      | rng.integers(0, 128, (45, 77)).astype(np.uint16),
        "all_patterns": workloads.all_patterns(),
        "random_bits": workloads.random_bits((300, 257), 6),
    }
    return out


SPECIALS = special_tensors()


@pytest.mark.parametrize("name", sorted(SPECIALS))
@pytest.mark.parametrize("geom", GEOMS[:4] + GEOMS[6:])
def test_roundtrip_special(name, geom):
    w = SPECIALS[name]
    blob = oracle.encode(w, *geom)
    assert oracle.validate(blob) == 0
    assert np.array_equal(oracle.decode(blob), w)


@pytest.mark.parametrize("geom", GEOMS)
def test_roundtrip_cfg1(geom):
    w = workloads.weights(1, "w")
    blob = oracle.encode(w, *geom)
    assert np.array_equal(oracle.decode(blob), w)


def test_encoding_is_deterministic():
    w = SPECIALS["127x1001"]
    a = oracle.encode(w, 16, 512, 64, 12)
    b = oracle.encode(w.copy(), 16, 512, 64, 12)
    assert np.array_equal(a, b)


def _chunk_block(h, tile, c):
    """Rows/cols of chunk c of `tile` by the geometry's definition."""
    TR, TC, S = h["tile_rows"], h["tile_cols"], h["chunks_per_tile"]
    V = TC // S
    n_tc = -(-h["cols"] // TC)
    ti, tj = divmod(tile, n_tc)
    r0, r1 = ti * TR, min(h["rows"], ti * TR + TR)
    tile_c1 = min(h["cols"], tj * TC + TC)
    c0 = min(tj * TC + c * V, tile_c1)
    c1 = min(c0 + V, tile_c1)
    return r0, r1, c0, c1


@pytest.mark.parametrize("geom", [(16, 512, 64, 12), (5, 24, 3, 11), (3, 7, 7, 10)])
def test_chunks_decode_alone_in_any_order(geom):
    w = SPECIALS["127x1001"]
    blob = oracle.encode(w, *geom)
    h = oracle.header(blob)
    e, _ = oracle.split(w)
    order = [(t, c) for t in range(h["n_tiles"]) for c in range(h["chunks_per_tile"])]
    rng = np.random.default_rng(0)
    rng.shuffle(order)
    for t, c in order[:400]:
        r0, r1, c0, c1 = _chunk_block(h, t, c)
        want = e[r0:r1, c0:c1].ravel()
        got = oracle.decode_chunk(blob, t, c)
        assert np.array_equal(got, want), (t, c)


def test_offsets_are_consistent():
    w = workloads.weights(1, "w")
    blob = oracle.encode(w, 16, 512, 64, 12)
    h = oracle.header(blob)
    sec = oracle.sections(blob)
    tw = sec["tile_words"].astype(np.int64)
    cb = sec["chunk_bits"].astype(np.int64).reshape(h["n_tiles"], h["chunks_per_tile"])
    assert tw[0] == 0 and tw[-1] == h["stream_words"]
    assert np.all(np.diff(tw) == (cb.sum(axis=1) + 31) // 32)
    # every section starts on a 256-byte boundary, in the documented order
    offs = [h[k] for k in ("off_code_len", "off_table", "off_tile_words", "off_chunk_bits",
                           "off_raw", "off_stream", "total_bytes")]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert h["total_bytes"] == blob.size
    # raw plane: row-major sign+fraction bytes, rows padded to 16 bytes with zeros
    _, r = oracle.split(w)
    assert np.array_equal(sec["raw"][:, : h["cols"]], r)
    assert h["raw_ld"] % 16 == 0 and np.all(sec["raw"][:, h["cols"]:] == 0)
    # the stored decode table is the one the stored lengths define
    assert np.array_equal(sec["table"], oracle.decode_table(sec["code_len"]))


def _bits_msb_first(codes, lens, syms):
    out = []
    for s in syms:
        c, l = int(codes[s]), int(lens[s])
        out.extend((c >> i) & 1 for i in range(l - 1, -1, -1))
    return out


def test_stream_bit_order_matches_deflate_convention():
    w = workloads.gaussian_bits((37, 53), 0.05, 9)
    blob = oracle.encode(w, 8, 16, 4, 12)
    h = oracle.header(blob)
    sec = oracle.sections(blob)
    lens = sec["code_len"]
    codes = oracle.canonical_codes(lens)
    words = sec["stream"]
    bits = ((words[:, None] >> np.arange(32, dtype=np.uint32)) & 1).ravel()
    e, _ = oracle.split(w)
    cb = sec["chunk_bits"].astype(np.int64).reshape(h["n_tiles"], h["chunks_per_tile"])
    for t in range(h["n_tiles"]):
        pos = int(sec["tile_words"][t]) * 32
        for c in range(h["chunks_per_tile"]):
            r0, r1, c0, c1 = _chunk_block(h, t, c)
            want = _bits_msb_first(codes, lens, e[r0:r1, c0:c1].ravel())
            n = int(cb[t, c])
            assert n == len(want)
            assert list(bits[pos:pos + n]) == want
            pos += n
        # padding to the next tile is zero
        end = int(sec["tile_words"][t + 1]) * 32
        assert not bits[pos:end].any()


def test_decode_table_entries():
    w = workloads.weights(1, "w")
    e, _ = oracle.split(w)
    lens = oracle.code_lengths(oracle.histogram(e), 12)
    codes = oracle.canonical_codes(lens)
    table = oracle.decode_table(lens)
    rev = {}
    for s in range(256):
        if lens[s]:
            l = int(lens[s])
            # the first stream bit (code MSB) sits in window bit 0
            r = int(format(int(codes[s]), "0%db" % l)[::-1], 2)
            rev[s] = (r, l)
    rng = np.random.default_rng(1)
    for win in rng.integers(0, 4096, 500):
        win = int(win)
        ent = int(table[win])
        s0 = [s for s, (r, l) in rev.items() if win & ((1 << l) - 1) == r]
        assert len(s0) == 1
        s0 = s0[0]
        l0 = rev[s0][1]
        rest = win >> l0
        s1 = [s for s, (r, l) in rev.items() if l <= 12 - l0 and rest & ((1 << l) - 1) == r]
        assert (ent >> 7) & 0xFF == s0 and (ent >> 16) & 0x7F == l0
        if s1:
            assert ent >> 31 == 0 and (ent >> 23) & 0xFF == s1[0]
            assert ent & 0xF == l0 + rev[s1[0]][1]
        else:
            assert ent >> 31 == 1 and ent & 0xF == l0 and (ent >> 23) & 0xFF == 0


# (tile rows, length limit, 6-bit cap of common exponents): the shipped
# default, the short-code variant, and the plain optimal code at limit 12
CODES = [(8, 8, 1024), (8, 6, 0), (16, 12, 0)]


@pytest.mark.parametrize("tr,lmax,pair_fit", CODES)
@pytest.mark.parametrize("cid,name", [(1, "w"), (2, "k"), (3, "k"), (3, "gate"), (5, "lm_head")])
def test_exponent_bits_within_one_bit_of_entropy(cid, name, tr, lmax, pair_fit):
    wl = workloads.WORKLOADS[cid]
    m = wl.matrix(name)
    rows = slice(0, min(m.rows, 1024))
    w = workloads.weights(cid, name, rows=rows)
    blob = oracle.encode(w, tr, 512, 64, lmax, pair_fit)
    e, _ = oracle.split(w)
    H = oracle.entropy_bits(oracle.histogram(e))
    rep = oracle.size_report(blob)
    assert rep["payload_bits_per_weight"] <= H + 1.0
    # including header, lengths, decode table, offsets and padding
    assert rep["exp_bits_per_weight"] <= H + 1.0, (rep, H)


def test_payload_within_huffman_bound_random_distributions():
    rng = np.random.default_rng(2)
    for trial in range(20):
        n = int(rng.integers(2, 256))
        p = rng.dirichlet(np.full(n, 0.3))
        syms = rng.choice(256, n, replace=False)
        e = rng.choice(syms, size=20000, p=p).astype(np.uint8)
        h = oracle.histogram(e)
        ln = oracle.code_lengths(h, 12)
        H = oracle.entropy_bits(h)
        avg = float((h * ln.astype(np.uint64)).sum()) / e.size
        assert H - 1e-9 <= avg <= H + 1.0


def _corrupt_cases(blob):
    h = oracle.header(blob)
    cases = {}
    b = blob.copy(); b[0] ^= 1; cases["magic"] = b
    b = blob.copy(); b[4] = 9; cases["version"] = b
    cases["truncated"] = blob[: blob.size - 300].copy()
    b = blob.copy(); b[h["off_table"] + 40] ^= 0x10; cases["table"] = b
    b = blob.copy(); b[h["off_chunk_bits"] + 6] ^= 0x01; cases["chunk_bits"] = b
    b = blob.copy(); b[h["off_tile_words"] + 8] ^= 0x01; cases["tile_words"] = b
    b = blob.copy(); lens = b[h["off_code_len"]: h["off_code_len"] + 256]
    nz = np.flatnonzero(lens)
    lens[nz[0]] = 1; lens[nz[1]] = 1; lens[nz[2]] = 1; cases["kraft"] = b
    b = blob.copy(); b[h["off_code_len"] + nz[0]] = 13; cases["too_long"] = b
    b = blob.copy(); b[8] ^= 0x01; cases["rows"] = b
    b = blob.copy(); b[28] = 0x07; cases["geometry"] = b
    return cases


def test_corrupted_blobs_rejected():
    w = SPECIALS["127x1001"]
    blob = oracle.encode(w, 16, 512, 64, 12)
    for name, bad in _corrupt_cases(blob).items():
        assert oracle.validate(bad) != 0, name
        with pytest.raises(ValueError):
            oracle.decode(bad)


def test_stream_corruption_detected_by_length_check():
    w = SPECIALS["127x1001"]
    blob = oracle.encode(w, 16, 512, 64, 12)
    h = oracle.header(blob)
    bad = blob.copy()
    # flip bits in the middle of the stream: the decoded chunk no longer ends at
    # its recorded length (or decodes to a different symbol)
    bad[h["off_stream"] + 100] ^= 0xFF
    try:
        got = oracle.decode(bad)
    except ValueError:
        return
    assert not np.array_equal(got, w)


def test_encode_rejects_bad_geometry():
    w = SPECIALS["1x1"]
    for geom in [(0, 512, 64, 12), (16, 500, 64, 12), (16, 512, 64, 13), (16, 512, 64, 5),
                 (512, 4096, 1, 12)]:
        with pytest.raises(ValueError):
            oracle.encode(w, *geom)


@pytest.mark.parametrize("lmax", [6, 7])
@pytest.mark.parametrize("tr", [8, 4])
def test_short_code_limits_round_trip(lmax, tr):
    # limits below 8 take tensors with at most 2^lmax distinct exponents
    for name in ("1x1", "one_symbol", "subnormal"):
        w = SPECIALS[name]
        assert np.array_equal(oracle.decode(oracle.encode(w, tr, 512, 64, lmax)), w)
    w = workloads.gaussian_bits((37, 1100), 0.02, 21)
    blob = oracle.encode(w, tr, 512, 64, lmax)
    assert oracle.header(blob)["max_code_len"] == lmax
    assert np.array_equal(oracle.decode(blob), w)


def test_short_code_limit_rejects_too_many_exponents():
    w = workloads.random_bits((64, 64), 3)          # all 256 exponent values
    for lmax in (6, 7):
        with pytest.raises(ValueError):
            oracle.encode(w, 8, 512, 64, lmax)
    assert np.array_equal(oracle.decode(oracle.encode(w, 8, 512, 64, 8)), w)
