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
