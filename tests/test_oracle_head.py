"""Pins for the oracle's head projection.

Z[r][v] = sum_k hidden[idx[r]][k] * W[v][k] (vllm-metal release v0.4.0,
Summary; mlxcel PR #1969: the head acts per position, so a gathered row's
logits equal the same row of the full projection).
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import ref_numpy


def test_integer_special_case_exact():
    """bf16 entries in {-4..4}: every product and partial sum is an exact
    integer, so the f64 result equals integer arithmetic exactly."""
    H, T, V = 96, 11, 300
    hid = synth.small_int_bf16(1, (T, H))
    w = synth.small_int_bf16(2, (V, H))
    idx = np.array([10, 0, 3, 3, 7], dtype=np.int32)
    Z = oracle.head(hid, w, idx)
    hi = synth.bf16_bits_to_f32(hid).astype(np.int64)
    wi = synth.bf16_bits_to_f32(w).astype(np.int64)
    exact = hi[idx] @ wi.T
    assert np.array_equal(Z, exact.astype(np.float64))


def test_one_hot_hidden_reads_weight_column():
    """A one-hot hidden row e_j gives Z[r][v] = W[v][j] exactly; catches a
    transposed operand or a wrong column index."""
    T, H, V = 6, 16, 40
    hid = np.zeros((T, H), dtype=np.float32)
    cols = [0, 5, 15, 7, 1, 9]
    for t, j in enumerate(cols):
        hid[t, j] = 1.0
    w = synth.normal_f32(synth.rng(3), (V, H))
    idx = np.arange(T, dtype=np.int32)
    Z = oracle.head(hid, w, idx)
    for t, j in enumerate(cols):
        assert np.array_equal(Z[t], w[:, j].astype(np.float64))


def test_selective_rows_equal_full_rows():
    """Selective rows equal the same rows of the full projection, bit for bit
    (vllm-metal release, Testing; mlxcel PR #1969); the shifted selection
    does not (the off-by-one control)."""
    d = synth.tiny_batch(1000)
    T = d["hidden"].shape[0]
    full = oracle.head(d["hidden"], d["weight"], np.arange(T, dtype=np.int32))
    st, idx, _ = oracle.rows(d["cu_seqlens"], d["num_decode"], T)
    assert st == oracle.OK
    sel = oracle.head(d["hidden"], d["weight"], idx)
    assert np.array_equal(sel, full[idx])
    shifted = np.clip(idx - 1, 0, T - 1)
    assert not np.array_equal(sel, full[shifted])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_head_vs_numpy_matmul(dtype):
    g = synth.rng(4)
    T, H, V = 13, 200, 257
    if dtype == "f32":
        hid, w = synth.normal_f32(g, (T, H)), synth.normal_f32(g, (V, H), 0.07)
    else:
        hid, w = synth.normal_bf16(g, (T, H)), synth.normal_bf16(g, (V, H), 0.07)
    idx = np.array([12, 0, 5, 5, 1], dtype=np.int32)
    Z = oracle.head(hid, w, idx)
    ref = ref_numpy.head(hid, w, idx)
    scale = np.abs(ref).max()
    assert np.max(np.abs(Z - ref)) <= 1e-12 * scale


def test_invalid_row_gives_nan():
    hid = np.ones((4, 8), dtype=np.float32)
    w = np.ones((5, 8), dtype=np.float32)
    Z = oracle.head(hid, w, np.array([0, 4, -1, 3], dtype=np.int32))
    assert np.all(Z[0] == 8.0) and np.all(Z[3] == 8.0)
    assert np.all(np.isnan(Z[1])) and np.all(np.isnan(Z[2]))


def _int_head(scale_mode=oracle.SCALE_NONE, scale=1.0, lib=None):
    hid = synth.small_int_bf16(31, (9, 80))
    w = synth.small_int_bf16(32, (50, 80))
    idx = np.array([8, 0, 5], dtype=np.int32)
    exact = (synth.bf16_bits_to_f32(hid).astype(np.int64)[idx]
             @ synth.bf16_bits_to_f32(w).astype(np.int64).T)
    return oracle.head(hid, w, idx, lib=lib, scale_mode=scale_mode, scale=scale), exact


def test_scale_modes_closed_forms():
    """Output scaling (vllm-metal release, Summary: Cohere's logit_scale,
    Granite's logits_scaling): none leaves the integer head; multiply by
    0.5 halves it exactly; divide by 4 quarters it exactly."""
    z, exact = _int_head()
    assert np.array_equal(z, exact.astype(np.float64))
    z, _ = _int_head(oracle.SCALE_MUL, 0.5)
    assert np.array_equal(z, exact / 2.0)
    z, _ = _int_head(oracle.SCALE_DIV, 4.0)
    assert np.array_equal(z, exact / 4.0)


def _div49_case(lib=None):
    """Integer head times 49 (the weights are 49 x small integers, exact in
    fp32), divided by 49."""
    hid = synth.small_int_bf16(33, (6, 64))
    wi = synth.bf16_bits_to_f32(synth.small_int_bf16(34, (40, 64)))
    w = (wi * np.float32(49.0)).astype(np.float32)
    idx = np.arange(6, dtype=np.int32)
    z = oracle.head(hid, w, idx, lib=lib, scale_mode=oracle.SCALE_DIV, scale=49.0)
    ints = synth.bf16_bits_to_f32(hid).astype(np.int64) @ wi.astype(np.int64).T
    return z, ints


def test_divide_is_a_true_division():
    """Dividing logits that are multiples of 49 by 49 returns the integers
    exactly; a multiply by the rounded reciprocal would miss some of them on
    this data (checked below), so the pin tells the two apart."""
    z, ints = _div49_case()
    assert np.array_equal(z, ints.astype(np.float64))
    recip = (ints * 49.0) * (1.0 / 49.0)
    assert not np.array_equal(recip, ints.astype(np.float64))
