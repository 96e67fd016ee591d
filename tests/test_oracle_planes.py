"""Pins for the oracle's BF16 interpretation and byte-plane split (CPU only).

The split is checked against facts that do not restate it: the BF16 definition
(golden examples from the data-types post), numpy's IEEE float32 reading of a
BF16 pattern placed in the top half of a float32, and algebraic invariants
(negation touches only the sign, doubling touches only the exponent).
"""
import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _golden_bf16():
    rows = []
    with open(os.path.join(GOLDEN, "bf16_examples.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            s, e, fr, val, _src = line.split()
            bits = (int(s, 2) << 15) | (int(e, 2) << 7) | int(fr, 2)
            rows.append((bits, float(val), int(e, 2), int(s, 2)))
    return rows


@pytest.mark.parametrize("bits,val,exp,sign", _golden_bf16())
def test_bf16_value_golden(bits, val, exp, sign):
    got = oracle.bf16_value(np.array([bits], np.uint16))[0]
    if math.isnan(val):
        assert math.isnan(got)
    else:
        assert got == val
        assert math.copysign(1.0, got) == math.copysign(1.0, val)
    e, r = oracle.split(np.array([bits], np.uint16))
    assert int(e[0]) == exp          # the exponent field is the coded byte
    assert int(r[0]) >> 7 == sign    # the sign travels in the raw byte's top bit


def test_bf16_value_matches_float32_top_half():
    # BF16 is the upper half of an IEEE float32; numpy's float32 reading is an
    # independent implementation of the same definition.
    with np.errstate(invalid="ignore"):
        ref = (ALL.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = oracle.bf16_value(ALL)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_split_join_exhaustive_roundtrip():
    e, r = oracle.split(ALL)
    assert np.array_equal(oracle.join(e, r), ALL)
    # the map is a bijection between 16-bit patterns and (e, r) byte pairs
    pairs = e.astype(np.uint32) * 256 + r
    assert np.unique(pairs).size == 65536


def test_split_negation_only_flips_raw_sign_bit():
    e, r = oracle.split(ALL)
    e2, r2 = oracle.split(ALL ^ np.uint16(0x8000))
    assert np.array_equal(e, e2)
    assert np.array_equal(r ^ r2, np.full(65536, 0x80, np.uint8))


def test_split_doubling_only_bumps_exponent():
    v = oracle.bf16_value(ALL)
    e, r = oracle.split(ALL)
    normal = (e >= 1) & (e <= 253)
    # the pattern of 2*v: take the float32 of 2*v, top half (exact for normals)
    doubled = ((v[normal] * 2).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    e2, r2 = oracle.split(doubled)
    assert np.array_equal(e2.astype(int), e[normal].astype(int) + 1)
    assert np.array_equal(r2, r[normal])


def test_raw_byte_entropy_near_eight_bits():
    # Sanity: on N(0, 0.02^2) weights the raw byte is close to uniform
    # (the NWC page reports 7.97 bits for trained weights).
    w = workloads.weights(1, "w")
    e, r = oracle.split(w)
    hr = np.bincount(r.ravel(), minlength=256)
    assert oracle.entropy_bits(hr) > 7.95


def test_histogram_counts_and_gaussian_binades():
    w = workloads.weights(1, "w")
    e, _ = oracle.split(w)
    h = oracle.histogram(e)
    n = w.size
    assert int(h.sum()) == n
    # Closed form: for |w| ~ half-normal(sigma), the mass of exponent e is
    # P(2^(e-127) <= |w| < 2^(e-126)).  Pool the tail bins and run a chi^2 test.
    from scipy.stats import chi2, norm
    sigma = 0.02
    es = np.arange(1, 255)
    lo, hi = 2.0 ** (es - 127), 2.0 ** (es - 126)
    p = 2 * (norm.cdf(hi / sigma) - norm.cdf(lo / sigma))
    obs = h[1:255].astype(np.float64)
    exp = p * n
    big = exp > 50
    o = np.append(obs[big], obs[~big].sum() + h[0] + h[255])
    x = np.append(exp[big], exp[~big].sum() + (n - exp.sum()))
    stat = float(((o - x) ** 2 / x).sum())
    dof = o.size - 1
    assert chi2.sf(stat, dof) > 1e-4, (stat, dof)
