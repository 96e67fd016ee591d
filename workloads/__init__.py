"""Seeded synthetic inputs for the five decode-GEMV workloads.

This module only draws random numbers and rounds them to BF16; it holds none
of the compression method's arithmetic.  It is the one module that both the
oracle-side tests and the product-side tests and benchmark import, so that
both sides see the same bits.

Recipe (every workload): z ~ N(0, 1) in float32 from numpy's PCG64, seeded by
SeedSequence([seed, workload, layer, matrix, stream]); w32 = z * sigma * s_row
(times 20 where an outlier mask is set); W = round-to-nearest-even to BF16 of
w32.  Row scales s_row = exp(U(ln lo, ln hi)) drawn once per matrix; outliers
are an independent Bernoulli mask.  Activations x ~ N(0, 1) rounded to BF16.
Everything is drawn in row blocks from one generator per stream, which yields
the same numbers as one draw of the whole matrix.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

STREAM_WEIGHTS, STREAM_ROWSCALE, STREAM_OUTLIER, STREAM_X = 0, 1, 2, 3


@dataclass(frozen=True)
class Matrix:
    name: str
    mid: int          # matrix id inside the workload
    rows: int         # N (outputs)
    cols: int         # K (inputs)


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    matrices: Tuple[Matrix, ...]
    layers: int
    sigma: float
    row_scale: Optional[Tuple[float, float]]
    outlier_p: float
    outlier_scale: float
    batches: Tuple[int, ...]
    # GEMVs that read the same activation vector in a decode step, in the
    # order the step runs them (used to group launches)
    groups: Tuple[Tuple[str, ...], ...] = field(default=())

    def weights_total(self) -> int:
        return self.layers * sum(m.rows * m.cols for m in self.matrices)

    def matrix(self, name: str) -> Matrix:
        for m in self.matrices:
            if m.name == name:
                return m
        raise KeyError(name)


def _qwen3_4b_layer() -> Tuple[Matrix, ...]:
    h, q, kv, f = 2560, 4096, 1024, 9728
    return (Matrix("q", 0, q, h), Matrix("k", 1, kv, h), Matrix("v", 2, kv, h),
            Matrix("o", 3, h, q), Matrix("gate", 4, f, h), Matrix("up", 5, f, h),
            Matrix("down", 6, h, f))


def _llama31_8b_layer() -> Tuple[Matrix, ...]:
    h, kv, f = 4096, 1024, 14336
    return (Matrix("q", 0, h, h), Matrix("k", 1, kv, h), Matrix("v", 2, kv, h),
            Matrix("o", 3, h, h), Matrix("gate", 4, f, h), Matrix("up", 5, f, h),
            Matrix("down", 6, h, f))


LAYER_GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))

WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "single_1024x1024", (Matrix("w", 0, 1024, 1024),), 1, 0.02, None, 0.0, 20.0,
                (1,), (("w",),)),
    2: Workload(2, "qwen3_4b_layer", _qwen3_4b_layer(), 1, 0.02, (0.5, 2.0), 0.0, 20.0, (1,),
                LAYER_GROUPS),
    3: Workload(3, "llama31_8b_step", _llama31_8b_layer(), 32, 0.02, None, 0.001, 20.0, (1,),
                LAYER_GROUPS),
    4: Workload(4, "skinny_4096x14336", (Matrix("w_4096x14336", 0, 4096, 14336),
                                         Matrix("w_14336x4096", 1, 14336, 4096)),
                1, 0.02, None, 0.0, 20.0, (2, 4, 8, 16), (("w_4096x14336",), ("w_14336x4096",))),
    5: Workload(5, "lm_head_128256x4096", (Matrix("lm_head", 0, 128256, 4096),), 1, 0.01,
                (0.25, 4.0), 0.0, 20.0, (1, 8), (("lm_head",),)),
}


def _rng(seed: int, cid: int, layer: int, mid: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cid, layer, mid, stream]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to BF16 (nearest, ties to even) and return the bit patterns.

    Finite inputs only (the generators never produce inf/NaN)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def weights(cid: int, name: str, layer: int = 0, seed: int = 0,
            rows: Optional[slice] = None, block_rows: int = 4096) -> np.ndarray:
    """BF16 bit patterns [N, K] of one matrix of a workload (uint16).

    ``rows`` selects a contiguous row range (the values are those of the full
    matrix: the generator is advanced past earlier rows)."""
    wl = WORKLOADS[cid]
    m = wl.matrix(name)
    N, K = m.rows, m.cols
    r0, r1 = (0, N) if rows is None else (rows.start or 0, rows.stop if rows.stop is not None else N)
    gz = _rng(seed, cid, layer, m.mid, STREAM_WEIGHTS)
    go = _rng(seed, cid, layer, m.mid, STREAM_OUTLIER) if wl.outlier_p > 0 else None
    scale = None
    if wl.row_scale is not None:
        lo, hi = wl.row_scale
        gs = _rng(seed, cid, layer, m.mid, STREAM_ROWSCALE)
        scale = np.exp(gs.uniform(np.log(lo), np.log(hi), size=N)).astype(np.float32)
    out = np.empty((r1 - r0, K), np.uint16)
    sigma = np.float32(wl.sigma)
    r = 0
    while r < r1:
        nb = min(block_rows, r1 - r)
        z = gz.standard_normal((nb, K), dtype=np.float32)
        mask = go.random((nb, K)) < wl.outlier_p if go is not None else None
        if r + nb > r0:
            w32 = z * sigma
            if scale is not None:
                w32 *= scale[r:r + nb, None]
            if mask is not None:
                w32[mask] *= np.float32(wl.outlier_scale)
            lo_i = max(r0 - r, 0)
            out[r + lo_i - r0: r + nb - r0] = f32_to_bf16_bits(w32[lo_i:])
        r += nb
    return out


def activations(cid: int, name: str, batch: int = 1, layer: int = 0, seed: int = 0) -> np.ndarray:
    """BF16 bit patterns [batch, K] ~ N(0, 1) for the matrix's input side."""
    wl = WORKLOADS[cid]
    m = wl.matrix(name)
    g = _rng(seed, cid, layer, m.mid, STREAM_X)
    return f32_to_bf16_bits(g.standard_normal((batch, m.cols), dtype=np.float32))


def all_patterns(rows: int = 256, cols: int = 256) -> np.ndarray:
    """Every one of the 65,536 BF16 bit patterns once, row-major (256 x 256)."""
    assert rows * cols == 65536
    return np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(rows, cols)


def random_bits(shape, seed: int) -> np.ndarray:
    """Uniformly random 16-bit patterns (every exponent, sign and fraction)."""
    g = np.random.default_rng(np.random.SeedSequence([seed, 99]))
    return g.integers(0, 65536, size=shape, dtype=np.uint32).astype(np.uint16)


def gaussian_bits(shape, sigma: float, seed: int) -> np.ndarray:
    """N(0, sigma^2) rounded to BF16, for ad-hoc shapes in tests."""
    g = np.random.default_rng(np.random.SeedSequence([seed, 98]))
    return f32_to_bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(sigma))
