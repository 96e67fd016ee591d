"""Pins for the oracle's FP64 matrix-vector and skinny matrix products (CPU).

Exact special cases: a one-hot x returns a column of W; one-hot rows of W
return entries of x; small integers give exact integer sums.  The general case
is compared with numpy's float64 matmul on the decoded values within the FP64
summation bound K * 2^-53 * sum|w x|.
"""
import numpy as np
import pytest

import oracle
import workloads


def _vals(bits):
    # BF16 -> float64 through numpy's float32 reading (pinned against the
    # definition in the planes tests)
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_one_hot_x_selects_a_column():
    w = workloads.gaussian_bits((37, 53), 0.02, 1)   # not square: a transpose would fail
    for k in [0, 7, 52]:
        x = np.zeros(53, np.uint16)
        x[k] = 0x3F80                                 # 1.0
        y, a = oracle.gemv(w, x)
        assert np.array_equal(y, _vals(w[:, k]))
        assert np.array_equal(a, np.abs(_vals(w[:, k])))


def test_one_hot_rows_select_x_entries():
    x = workloads.gaussian_bits((64,), 1.0, 2)
    w = np.zeros((10, 64), np.uint16)
    for n in range(10):
        w[n, (7 * n) % 64] = 0xBF80                   # -1.0
    y, _ = oracle.gemv(w, x)
    assert np.array_equal(y, -_vals(x[(7 * np.arange(10)) % 64]))


def test_small_integers_exact():
    rng = np.random.default_rng(3)
    wi = rng.integers(-8, 9, (20, 300))
    xi = rng.integers(-8, 9, 300)
    wb = workloads.f32_to_bf16_bits(wi.astype(np.float32))
    xb = workloads.f32_to_bf16_bits(xi.astype(np.float32))
    y, a = oracle.gemv(wb, xb)
    assert np.array_equal(y, (wi @ xi).astype(np.float64))
    assert np.array_equal(a, (np.abs(wi) @ np.abs(xi)).astype(np.float64))


def test_matches_numpy_within_fp64_bound():
    w = workloads.weights(1, "w")[:200]
    x = workloads.activations(1, "w")[0]
    y, a = oracle.gemv(w, x)
    ref = _vals(w) @ _vals(x)
    K = w.shape[1]
    assert np.all(np.abs(y - ref) <= 2 * K * 2.0 ** -53 * a)
    assert np.all(np.abs(y) <= a)


def test_subnormal_weights_kept():
    # an all-subnormal row: the products are tiny but exact in FP64
    w = np.array([[0x0001, 0x0040, 0x8002, 0x007F]], np.uint16)
    x = workloads.f32_to_bf16_bits(np.array([1.0, 2.0, 4.0, -0.5], np.float32))
    y, _ = oracle.gemv(w, x)
    want = (1 * 1.0 + 64 * 2.0 - 2 * 4.0 + 127 * -0.5) * 2.0 ** -133
    assert y[0] == want


def test_gemm_is_rowwise_gemv():
    w = workloads.gaussian_bits((33, 70), 0.02, 4)
    X = workloads.gaussian_bits((5, 70), 1.0, 5)
    Y, A = oracle.gemm(w, X)
    for b in range(5):
        y, a = oracle.gemv(w, X[b])
        assert np.array_equal(Y[b], y) and np.array_equal(A[b], a)
    ref = _vals(X) @ _vals(w).T
    assert np.all(np.abs(Y - ref) <= 2 * 70 * 2.0 ** -53 * A)


def test_gemv_rows_subset():
    w = workloads.gaussian_bits((50, 40), 0.02, 6)
    x = workloads.gaussian_bits((40,), 1.0, 7)
    y, a = oracle.gemv(w, x)
    idx = np.array([3, 17, 49])
    ys, as_ = oracle.gemv_rows(w, x, idx)
    assert np.array_equal(ys, y[idx]) and np.array_equal(as_, a[idx])


def test_decoded_blob_feeds_gemv():
    w = workloads.gaussian_bits((100, 130), 0.02, 8)
    x = workloads.gaussian_bits((130,), 1.0, 9)
    blob = oracle.encode(w, 16, 64, 8, 12)
    y1, _ = oracle.gemv(oracle.decode(blob), x)
    y0, _ = oracle.gemv(w, x)
    assert np.array_equal(y0, y1)
