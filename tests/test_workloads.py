"""The seeded input generators: shapes, reproducibility, BF16 rounding (CPU)."""
import numpy as np
import pytest
import torch

import workloads


def test_shapes():
    wl = workloads.WORKLOADS
    assert [(m.rows, m.cols) for m in wl[2].matrices] == [
        (4096, 2560), (1024, 2560), (1024, 2560), (2560, 4096), (9728, 2560), (9728, 2560),
        (2560, 9728)]
    assert wl[3].layers == 32 and wl[3].weights_total() == 32 * (
        2 * 4096 * 4096 + 2 * 1024 * 4096 + 3 * 14336 * 4096)
    assert wl[5].matrices[0].rows == 128256 and wl[4].batches == (2, 4, 8, 16)


def test_blockwise_equals_whole():
    a = workloads.weights(2, "k", block_rows=1024)
    b = workloads.weights(2, "k", block_rows=37)
    assert np.array_equal(a, b)
    c = workloads.weights(2, "k", rows=slice(100, 333), block_rows=64)
    assert np.array_equal(a[100:333], c)
    o1 = workloads.weights(3, "k", block_rows=1024)
    o2 = workloads.weights(3, "k", block_rows=100)
    assert np.array_equal(o1, o2)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    f = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 0.02,
                        np.array([1.0, -2.5, 1e-40, -1e-39, 3.0e38], np.float32)])
    ours = workloads.f32_to_bf16_bits(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_distributions():
    w = workloads.weights(3, "k")
    v = (w.astype(np.uint32) << 16).view(np.float32)
    big = np.abs(v) > 0.2                       # > 10 sigma: essentially the 20x outliers
    assert 0.0003 < big.mean() < 0.0015
    w5 = workloads.weights(5, "lm_head", rows=slice(0, 2000))
    v5 = (w5.astype(np.uint32) << 16).view(np.float32)
    rs = v5.std(axis=1) / 0.01
    assert 0.2 < rs.min() < 0.35 and 3.0 < rs.max() < 4.5
    x = workloads.activations(2, "q", batch=3)
    assert x.shape == (3, 2560)


def test_distinct_layers_and_matrices():
    a = workloads.weights(3, "k", layer=0)
    b = workloads.weights(3, "k", layer=1)
    assert not np.array_equal(a, b)
