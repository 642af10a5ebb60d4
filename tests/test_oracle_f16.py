"""Pins for the oracle's f16 logits (MTPLX PR #532, Tests: parity on
synthetic bf16/f16 logits): the exact f64 value of every IEEE binary16 bit
pattern, and the reduction of f16 rows against the same rows given as f64."""
import math

import numpy as np

import oracle
import synth


def test_every_f16_pattern_widens_exactly():
    """All 65,536 bit patterns against numpy's float16 -> float64 conversion:
    normals, subnormals, signed zeros, infinities; NaNs stay NaN."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = bits.view(np.float16)
    got = oracle.widen(h)
    want = h.astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_f16_closed_forms():
    """Hand values: 1.0 = 0x3C00, -2.0 = 0xC000, 65504 = 0x7BFF (largest
    normal), 2^-14 = 0x0400 (smallest normal), 2^-24 = 0x0001 (smallest
    subnormal)."""
    bits = np.array([0x3C00, 0xC000, 0x7BFF, 0x0400, 0x0001, 0x8000], dtype=np.uint16)
    got = oracle.widen(bits.view(np.float16))
    assert got.tolist()[:5] == [1.0, -2.0, 65504.0, 2.0 ** -14, 2.0 ** -24]
    assert got[5] == 0.0 and math.copysign(1.0, got[5]) == -1.0


def test_f16_rows_reduce_like_their_f64_values():
    g = synth.rng(61)
    x = (g.standard_normal((5, 1000)) * 3).astype(np.float16)
    x[1, ::7] = -np.inf
    sel = g.integers(0, 1000, size=5).astype(np.int32)
    a = oracle.reduce(x, sel, 9)
    b = oracle.reduce(x.astype(np.float64), sel, 9)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
