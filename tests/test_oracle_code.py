"""Pins for the oracle's code construction (CPU only).

* package-merge lengths equal the brute-force optimum over every admissible
  length vector on small alphabets, including limits that bind;
* without a binding limit the cost equals a textbook heap Huffman code;
* canonical codes reproduce RFC 1951's worked example;
* zlib (an independent DEFLATE decoder) decodes a DEFLATE block built from the
  oracle's lengths, canonical codes and bit packing, which pins all three.
"""
import heapq
import itertools
import os
import zlib

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hist(counts):
    h = np.zeros(256, np.uint64)
    for s, c in counts.items():
        h[s] = c
    return h


def _cost(h, ln):
    return int((h.astype(np.int64) * ln.astype(np.int64)).sum())


def _brute_min(counts, L):
    syms = sorted(counts)
    c = np.array([counts[s] for s in syms], np.int64)
    best = None
    n = len(syms)
    grids = np.array(list(itertools.product(range(1, L + 1), repeat=n)), np.int64)
    kraft = (2.0 ** (-grids)).sum(axis=1)
    ok = kraft <= 1.0 + 1e-12
    costs = grids[ok] @ c
    return int(costs.min())


def _heap_huffman_cost(counts):
    if len(counts) == 1:
        return list(counts.values())[0]
    heap = [(c, i) for i, c in enumerate(counts.values())]
    heapq.heapify(heap)
    total = 0
    k = len(heap)
    while len(heap) > 1:
        a, _ = heapq.heappop(heap)
        b, _ = heapq.heappop(heap)
        total += a + b
        heapq.heappush(heap, (a + b, k))
        k += 1
    return total


CASES = []
_rng = np.random.default_rng(1234)
for n in range(2, 8):
    for trial in range(3):
        kind = trial % 3
        if kind == 0:
            cnt = _rng.integers(1, 100, n)
        elif kind == 1:
            cnt = (2 ** np.arange(n))[::-1] * _rng.integers(1, 3, n)   # geometric: deep tree
        else:
            cnt = np.maximum(1, (1000 * _rng.random(n) ** 4).astype(int))
        syms = _rng.choice(256, n, replace=False)
        counts = {int(s): int(c) for s, c in zip(syms, cnt)}
        lmin = int(np.ceil(np.log2(n)))
        for L in range(max(lmin, 1), 7 if n <= 6 else 6):
            CASES.append((counts, L))


@pytest.mark.parametrize("counts,L", CASES)
def test_package_merge_is_optimal(counts, L):
    h = _hist(counts)
    ln = oracle.code_lengths(h, L)
    assert all(ln[s] > 0 for s in counts)
    assert all(ln[s] == 0 for s in range(256) if s not in counts)
    assert int(ln.max()) <= L
    kraft = sum(2.0 ** -int(ln[s]) for s in counts)
    assert abs(kraft - 1.0) < 1e-12           # complete code for n >= 2
    assert _cost(h, ln) == _brute_min(counts, L)


def test_package_merge_equals_heap_huffman_when_limit_is_loose():
    rng = np.random.default_rng(7)
    for trial in range(40):
        n = int(rng.integers(2, 60))
        syms = rng.choice(256, n, replace=False)
        cnt = rng.integers(1, 10000, n)
        counts = {int(s): int(c) for s, c in zip(syms, cnt)}
        h = _hist(counts)
        ln = oracle.code_lengths(h, 30)
        assert _cost(h, ln) == _heap_huffman_cost(counts)


def test_code_lengths_degenerate_alphabets():
    h = np.zeros(256, np.uint64)
    with pytest.raises(ValueError):
        oracle.code_lengths(h, 12)
    h[77] = 5
    ln = oracle.code_lengths(h, 12)
    assert ln[77] == 1 and ln.sum() == 1
    h = np.ones(256, np.uint64)
    ln = oracle.code_lengths(h, 8)
    assert np.all(ln == 8)
    with pytest.raises(ValueError):
        oracle.code_lengths(h, 7)     # 256 symbols cannot fit in 7 bits


def test_canonical_codes_rfc1951_example():
    lens = np.zeros(256, np.uint8)
    want = {}
    with open(os.path.join(GOLDEN, "rfc1951_canonical.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            s, l, c = line.split()
            lens[int(s)] = int(l)
            want[int(s)] = c
    codes = oracle.canonical_codes(lens)
    for s, c in want.items():
        assert format(int(codes[s]), "0%db" % int(lens[s])) == c


def test_canonical_codes_prefix_free_and_ordered():
    rng = np.random.default_rng(3)
    for trial in range(30):
        n = int(rng.integers(2, 200))
        syms = rng.choice(256, n, replace=False)
        h = np.zeros(256, np.uint64)
        h[syms] = rng.integers(1, 1 << 20, n)
        ln = oracle.code_lengths(h, 12)
        codes = oracle.canonical_codes(ln)
        strs = {int(s): format(int(codes[s]), "0%db" % int(ln[s])) for s in syms}
        vals = sorted(strs.values())
        for a, b in zip(vals, vals[1:]):
            assert not b.startswith(a)
        # codes of one length are consecutive in symbol order
        order = sorted(strs, key=lambda s: (ln[s], s))
        left = [int(strs[s].ljust(12, "0"), 2) for s in order]
        assert left == sorted(left) and len(set(left)) == len(left)


def test_oversubscribed_lengths_rejected():
    ln = np.zeros(256, np.uint8)
    ln[:3] = 1
    with pytest.raises(ValueError):
        oracle.canonical_codes(ln)


# ---------------------------------------------------------------- zlib pin --

class _BitWriter:
    """LSB-first bit writer; DEFLATE header numbers go LSB first, Huffman
    codes MSB first (RFC 1951 section 3.1.1)."""

    def __init__(self):
        self.bits = []

    def number(self, value, n):
        for i in range(n):
            self.bits.append((value >> i) & 1)

    def code(self, value, n):
        for i in range(n - 1, -1, -1):
            self.bits.append((value >> i) & 1)

    def tobytes(self):
        out = bytearray()
        for i in range(0, len(self.bits), 8):
            b = 0
            for j, bit in enumerate(self.bits[i:i + 8]):
                b |= bit << j
            out.append(b)
        return bytes(out)


@pytest.mark.parametrize("src", ["cfg1", "skewed", "uniform200"])
def test_zlib_decodes_oracle_codes(src):
    rng = np.random.default_rng(11)
    if src == "cfg1":
        e, _ = oracle.split(workloads.weights(1, "w")[:64])
        data = bytes(e.ravel())
    elif src == "skewed":
        data = bytes((rng.geometric(0.35, 20000) % 200).astype(np.uint8))
    else:
        data = bytes(rng.integers(0, 200, 20000).astype(np.uint8))
    h = np.bincount(np.frombuffer(data, np.uint8), minlength=256)
    # The end-of-block symbol (256) needs a code.  Give its weight to byte 255,
    # which the data never uses: 255 is then the last symbol of its length in
    # canonical order, so renaming it 256 leaves every other code unchanged and
    # hands 256 exactly the code the oracle built for 255.
    assert h[255] == 0
    blk = _deflate_block_with_slot(data, 12, 255)
    assert zlib.decompress(blk, wbits=-15) == data


def _deflate_block_with_slot(data, lmax, slot):
    """One final dynamic-Huffman DEFLATE block carrying `data` as literals,
    coded with the oracle's lengths, canonical codes and MSB-first code order."""
    h = np.bincount(np.frombuffer(data, np.uint8), minlength=256).astype(np.uint64)
    h[slot] = 1
    ln = oracle.code_lengths(h, lmax)
    codes = oracle.canonical_codes(ln)
    lit_len = [int(ln[s]) for s in range(256)] + [int(ln[slot])]
    lit_len[slot] = 0
    w = _BitWriter()
    w.number(1, 1)        # BFINAL
    w.number(2, 2)        # BTYPE = dynamic Huffman
    w.number(0, 5)        # HLIT: 257 literal/length codes
    w.number(0, 5)        # HDIST: 1 distance code
    w.number(15, 4)       # HCLEN: all 19 code-length codes
    # code-length alphabet: symbols 0..15 all get 4-bit codes, so the canonical
    # code of symbol l is l itself; 16, 17, 18 are unused
    for s in [16, 17, 18, 0, 8, 7, 9, 6, 10, 5, 11, 4, 12, 3, 13, 2, 14, 1, 15]:
        w.number(4 if s < 16 else 0, 3)
    for l in lit_len:
        w.code(l, 4)
    w.code(1, 4)          # the single distance code has length 1
    for b in data:
        w.code(int(codes[b]), int(ln[b]))
    # symbol 256 takes the code the oracle gave to `slot` (same length, and the
    # next value in canonical order because slot was the last of its length)
    w.code(int(codes[slot]), int(ln[slot]))
    return w.tobytes()


def _brute_min_capped(counts, caps):
    # every length vector with l_s <= caps[s] under Kraft's inequality
    syms = sorted(counts)
    c = np.array([counts[s] for s in syms], np.int64)
    grids = np.array(list(itertools.product(*[range(1, caps[s] + 1) for s in syms])), np.int64)
    ok = (2.0 ** (-grids)).sum(axis=1) <= 1.0 + 1e-12
    return int((grids[ok] @ c).min())


PAIR_FIT_CASES = []
_rng2 = np.random.default_rng(4321)
for n in range(2, 8):
    for trial in range(4):
        cnt = np.maximum(1, (10000 * _rng2.random(n) ** 6).astype(int))    # a few heavy, several light
        syms = _rng2.choice(256, n, replace=False)
        PAIR_FIT_CASES.append(({int(s): int(c) for s, c in zip(syms, cnt)}, int(_rng2.choice([4, 16, 64]))))


@pytest.mark.parametrize("counts,pair_fit", PAIR_FIT_CASES)
def test_pair_fit_lengths_are_optimal_under_their_caps(counts, pair_fit):
    # lmax 8; symbols with count * pair_fit >= total are capped at 6 bits
    h = _hist(counts)
    total = sum(counts.values())
    caps = {s: (6 if c * pair_fit >= total else 8) for s, c in counts.items()}
    ln = oracle.code_lengths(h, 8, pair_fit)
    assert all(0 < ln[s] <= caps[s] for s in counts)
    assert abs(sum(2.0 ** -int(ln[s]) for s in counts) - 1.0) < 1e-12
    assert _cost(h, ln) == _brute_min_capped(counts, caps)


def test_pair_fit_zero_is_the_plain_limit_and_caps_can_be_infeasible():
    rng = np.random.default_rng(9)
    h = np.zeros(256, np.uint64)
    h[rng.choice(256, 40, replace=False)] = rng.integers(1, 10 ** 6, 40)
    assert np.array_equal(oracle.code_lengths(h, 8, 0), oracle.code_lengths(h, 8))
    # 65 equally common symbols all capped at 6 bits cannot form a prefix code:
    # the plain limit applies instead
    h = np.zeros(256, np.uint64)
    h[:65] = 1000
    assert np.array_equal(oracle.code_lengths(h, 8, 65), oracle.code_lengths(h, 8))
    assert int(oracle.code_lengths(h, 8, 65).max()) == 7


# -------------------------------------------- ranked unary code with escape --
# ("NWC -- Neural Weight Compression", How it works, bullet "Prefix code
# instead of rANS": exponents ranked by frequency, a unary rank code, an
# escape for rare values; the escape carries an index into the escaped
# symbols so every code fits the length limit)

def test_unary_worked_example_by_hand():
    # counts 1000, 500, 250 and ten symbols of 10 (1850 in all), lmax 8.
    # Cost of R unary ranks (rank r: r + 1 bits) plus an escape of R bits and
    # a ceil(log2(13 - R))-bit index for the rest, worked out by hand:
    #   R = 0: 13 escaped, 4-bit index          1850 * 4               = 7400
    #   R = 1: 12 escaped, 5 bits               1000 + 850 * 5         = 5250
    #   R = 2: 11 escaped, 6 bits               1000 + 1000 + 350 * 6  = 4100
    #   R = 3: 10 escaped, 7 bits               1000 + 1000 + 750 + 700 = 3450
    #   R = 4:  9 escaped, 8 bits               2750 + 40 + 90 * 8     = 3510
    #   R = 5:  8 escaped, 8 bits               2750 + 40 + 50 + 640   = 3480
    #   R >= 6: escapes over 8 bits, not allowed
    # so R = 3: lengths 1, 2, 3 and 7 for the ten rare symbols.
    counts = {10: 1000, 20: 500, 30: 250}
    counts.update({s: 10 for s in range(40, 50)})
    h = _hist(counts)
    ln = oracle.code_lengths_unary(h, 8)
    assert (ln[10], ln[20], ln[30]) == (1, 2, 3)
    assert all(ln[s] == 7 for s in range(40, 50))
    assert int(sum(int(h[s]) * int(ln[s]) for s in counts)) == 3450
    assert int(np.count_nonzero(ln)) == 13
    # the canonical code is the unary code, then the escape prefix 111 and a
    # 4-bit index in symbol order: 0, 10, 110, 1110000 .. 1111001
    code = oracle.canonical_codes(ln)
    assert (int(code[10]), int(code[20]), int(code[30])) == (0b0, 0b10, 0b110)
    assert [int(code[s]) for s in range(40, 50)] == [0b1110000 + i for i in range(10)]


def test_unary_is_optimal_for_dyadic_geometric_counts():
    # counts halving rank by rank: the unary code is a Huffman code and its
    # cost equals the entropy exactly (lengths 1 .. 7, 7)
    counts = {3 * i + 1: 2 ** (6 - i) for i in range(7)}
    counts[200] = 1
    h = _hist(counts)
    ln = oracle.code_lengths_unary(h, 12)
    assert [int(ln[3 * i + 1]) for i in range(7)] == list(range(1, 8)) and int(ln[200]) == 7
    n = sum(counts.values())
    H = oracle.entropy_bits(h) * n
    assert abs(_cost(h, ln) - H) < 1e-9
    assert _cost(h, ln) == _cost(h, oracle.code_lengths(h, 12))


@pytest.mark.parametrize("lmax", [8, 10, 12])
def test_unary_never_beats_the_length_limited_optimum(lmax):
    # the package-merge lengths are optimal among all prefix codes of at most
    # lmax bits, and the unary code is one of them: never cheaper, always a
    # prefix code, lengths by rank
    rng = np.random.default_rng(77 + lmax)
    for trial in range(40):
        n = int(rng.integers(2, 40))
        syms = rng.choice(256, n, replace=False)
        cnt = np.maximum(1, (10 ** 6 * rng.random(n) ** 4).astype(np.int64))
        h = np.zeros(256, np.uint64)
        h[syms] = cnt
        lu = oracle.code_lengths_unary(h, lmax)
        lh = oracle.code_lengths(h, lmax)
        assert _cost(h, lh) <= _cost(h, lu)
        present = np.flatnonzero(h)
        assert np.all(lu[present] >= 1) and np.all(lu[present] <= lmax)
        assert sum(2.0 ** -int(lu[s]) for s in present) <= 1.0 + 1e-12
        # more frequent symbols never get longer codes (ties by symbol)
        order = sorted(present, key=lambda s: (-int(h[s]), int(s)))
        assert all(int(lu[a]) <= int(lu[b]) for a, b in zip(order, order[1:]))


def test_unary_one_symbol_and_round_trip():
    h = np.zeros(256, np.uint64)
    h[127] = 5
    ln = oracle.code_lengths_unary(h, 8)
    assert int(ln[127]) == 1 and int(np.count_nonzero(ln)) == 1
    for w in (workloads.weights(1, "w", rows=slice(0, 200)), workloads.all_patterns(),
              workloads.gaussian_bits((37, 1001), 0.05, 3)):
        for lmax in (8, 12):
            blob = oracle.encode(w, 8, 512, 64, lmax, 0, family=1)
            assert oracle.validate(blob) == 0
            assert np.array_equal(oracle.decode(blob), w)
